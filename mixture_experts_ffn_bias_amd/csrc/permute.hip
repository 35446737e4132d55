// Token counting and expert-contiguous order ("DeepSeek-V3.2-Exp · MoE update",
// moe-forward excerpt: bincount of the selected experts, then for each expert
// the tokens that chose it in ascending token order), and the FP8 quantisation
// of x that the expert Linear layers consume.
//
// The order is built without atomics on global memory and without a host
// round trip: each 256-token chunk marks, per expert, which of its tokens
// chose it (a 256-bit mask in LDS); the popcount of the mask gives the chunk's
// count and, below a token's bit, that token's rank.  A single-workgroup scan
// turns chunk counts into per-chunk bases, so every (token, choice) pair gets
// its final row directly and the order is deterministic.
#include "common.h"
#include "kernels.h"
#include "plan.h"

namespace moe {

namespace {

constexpr int MASK_WORDS = PERM_CHUNK / 32;

__device__ __forceinline__ int clamp_expert(int e, int E) { return e < 0 ? 0 : (e >= E ? E - 1 : e); }

__device__ __forceinline__ void build_masks(uint32_t* mask, const int32_t* idx, int T, int K, int E) {
  for (int i = threadIdx.x; i < E * MASK_WORDS; i += blockDim.x) mask[i] = 0u;
  __syncthreads();
  const int t = blockIdx.x * PERM_CHUNK + threadIdx.x;
  if (t < T) {
    for (int k = 0; k < K; ++k) {
      const int e = clamp_expert(idx[(size_t)t * K + k], E);
      atomicOr(&mask[e * MASK_WORDS + (threadIdx.x >> 5)], 1u << (threadIdx.x & 31));
    }
  }
  __syncthreads();
}

// grid = chunks, block = PERM_CHUNK
__global__ __launch_bounds__(PERM_CHUNK) void count_kernel(const int32_t* __restrict__ idx, int T, int K, int E,
                                                          int32_t* __restrict__ chunk_cnt) {
  __shared__ uint32_t mask[256 * MASK_WORDS];
  build_masks(mask, idx, T, K, E);
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int c = 0;
#pragma unroll
    for (int j = 0; j < MASK_WORDS; ++j) c += __popc(mask[e * MASK_WORDS + j]);
    chunk_cnt[(size_t)blockIdx.x * E + e] = c;
  }
}

// one block of 256 threads; thread e walks the chunks of expert e
__global__ __launch_bounds__(256) void scan_kernel(const int32_t* __restrict__ chunk_cnt, int nchunks, int E,
                                                   int32_t* __restrict__ chunk_off, int32_t* __restrict__ counts,
                                                   int32_t* __restrict__ offsets) {
  __shared__ int s[256];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    for (int c = 0; c < nchunks; ++c) {
      chunk_off[(size_t)c * E + e] = run;
      run += chunk_cnt[(size_t)c * E + e];
    }
  }
  s[e] = run;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {  // inclusive Hillis-Steele scan
    const int v = e >= o ? s[e - o] : 0;
    __syncthreads();
    s[e] += v;
    __syncthreads();
  }
  if (e < E) {
    counts[e] = run;
    offsets[e] = s[e] - run;
  }
  if (e == E - 1) offsets[E] = s[e];
}

// grid = chunks, block = PERM_CHUNK
__global__ __launch_bounds__(PERM_CHUNK) void scatter_kernel(const int32_t* __restrict__ idx, int T, int K, int E,
                                                            const int32_t* __restrict__ chunk_off,
                                                            const int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ row_token,
                                                            int32_t* __restrict__ pair_row) {
  __shared__ uint32_t mask[256 * MASK_WORDS];
  build_masks(mask, idx, T, K, E);
  const int t = blockIdx.x * PERM_CHUNK + threadIdx.x;
  if (t >= T) return;
  const int w = threadIdx.x >> 5;
  const uint32_t below = (1u << (threadIdx.x & 31)) - 1u;
  for (int k = 0; k < K; ++k) {
    const int e = clamp_expert(idx[(size_t)t * K + k], E);
    const uint32_t* m = mask + e * MASK_WORDS;
    int rank = __popc(m[w] & below);
    for (int j = 0; j < w; ++j) rank += __popc(m[j]);
    const int pos = offsets[e] + chunk_off[(size_t)blockIdx.x * E + e] + rank;
    row_token[pos] = t;
    pair_row[(size_t)t * K + k] = pos;
  }
  row_token[(size_t)T * K + t] = t;  // the shared expert's rows: identity
}

// Per-128-block e4m3 quantisation of bf16 rows: 8 lanes per block, 16
// elements per lane.  scale = amax / 448 (correctly rounded fp32 division),
// code = e4m3_rne(v / scale); an all-zero block gets scale 1.  The 8 lanes
// of a block are consecutive lanes of one wave and call this together.
__device__ __forceinline__ void quant_block(const uint16_t* __restrict__ x, int64_t blk, int sub,
                                            uint8_t* __restrict__ q, float* __restrict__ scale) {
  const uint4* p = (const uint4*)(x + blk * BLK + sub * 16);
  const uint4 u0 = p[0], u1 = p[1];
  const uint32_t w[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
  float v[16];
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    v[2 * j] = bf16_to_f32(w[j] & 0xFFFFu);
    v[2 * j + 1] = bf16_to_f32(w[j] >> 16);
    amax = fmaxf(amax, fmaxf(fabsf(v[2 * j]), fabsf(v[2 * j + 1])));
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  amax = fmaxf(amax, __shfl_xor(amax, 4));
  const float sc = amax == 0.f ? 1.f : amax / E4M3_MAX;
  uint4 o;
  o.x = pack4_e4m3(v[0] / sc, v[1] / sc, v[2] / sc, v[3] / sc);
  o.y = pack4_e4m3(v[4] / sc, v[5] / sc, v[6] / sc, v[7] / sc);
  o.z = pack4_e4m3(v[8] / sc, v[9] / sc, v[10] / sc, v[11] / sc);
  o.w = pack4_e4m3(v[12] / sc, v[13] / sc, v[14] / sc, v[15] / sc);
  *(uint4*)(q + blk * BLK + sub * 16) = o;
  if (sub == 0) scale[blk] = sc;
}

__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ x, int64_t nblocks,
                                                         uint8_t* __restrict__ q, float* __restrict__ scale) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t blk = gid >> 3;
  if (blk >= nblocks) return;  // whole 8-lane groups leave together
  quant_block(x, blk, (int)(gid & 7), q, scale);
}

// Everything for T <= PERM_CHUNK in one launch: block 0 counts, scans and
// scatters (one chunk, masks kept in LDS); blocks 1.. quantise x.
__global__ __launch_bounds__(PERM_CHUNK) void permute_small_kernel(
    const int32_t* __restrict__ idx, int T, int K, int E, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ row_token, int32_t* __restrict__ pair_row,
    const uint16_t* __restrict__ x, int64_t nblocks, uint8_t* __restrict__ q, float* __restrict__ scale,
    PlanArgs plan) {
  if (blockIdx.x > 0) {
    const int64_t gid = (int64_t)(blockIdx.x - 1) * blockDim.x + threadIdx.x;
    const int64_t blk = gid >> 3;
    if (blk < nblocks) quant_block(x, blk, (int)(gid & 7), q, scale);
    return;
  }
  __shared__ uint32_t mask[256 * MASK_WORDS];
  __shared__ int s[256];
  __shared__ int s_off[256];
  build_masks(mask, idx, T, K, E);
  const int e = threadIdx.x;
  int cnt = 0;
  if (e < E) {
#pragma unroll
    for (int j = 0; j < MASK_WORDS; ++j) cnt += __popc(mask[e * MASK_WORDS + j]);
  }
  s[e] = cnt;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int v = e >= o ? s[e - o] : 0;
    __syncthreads();
    s[e] += v;
    __syncthreads();
  }
  s_off[e] = s[e] - cnt;
  if (e < E) {
    counts[e] = cnt;
    offsets[e] = s[e] - cnt;
  }
  if (e == 255) offsets[E] = s[255];
  __syncthreads();
  const int t = threadIdx.x;
  if (t < T) {
    const int w = t >> 5;
    const uint32_t below = (1u << (t & 31)) - 1u;
    for (int k = 0; k < K; ++k) {
      const int ek = clamp_expert(idx[(size_t)t * K + k], E);
      const uint32_t* m = mask + ek * MASK_WORDS;
      int rank = __popc(m[w] & below);
      for (int j = 0; j < w; ++j) rank += __popc(m[j]);
      const int pos = s_off[ek] + rank;
      row_token[pos] = t;
      pair_row[(size_t)t * K + k] = pos;
    }
    row_token[(size_t)T * K + t] = t;
  }
  if (plan.tiles) {  // the FFN tile list from the same offsets
    __syncthreads();  // s is reused as the plan's scan buffer
    plan_tiles_block(e < E ? s_off[e] : 0, e < E ? cnt : 0, T, K, plan.tile_rows, plan.has_shared, plan.cap, 0, E, s,
                     plan.tiles, plan.n_tiles);
  }
}

}  // namespace

hipError_t launch_quant(const uint16_t* x, int64_t T, int d, uint8_t* xq, float* xs, hipStream_t s) {
  const int64_t nblocks = T * (d / BLK);
  const int64_t threads = nblocks * 8;
  hipLaunchKernelGGL(quant_rows_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, x, nblocks, xq, xs);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* idx, const uint16_t* x, int T, int d, int E, int K, int32_t* chunk_cnt,
                          int32_t* chunk_off, int32_t* counts, int32_t* offsets, int32_t* row_token,
                          int32_t* pair_row, uint8_t* xq, float* xs, hipStream_t s, const PlanArgs* plan,
                          bool* planned) {
  const int nchunks = (T + PERM_CHUNK - 1) / PERM_CHUNK;
  if (planned) *planned = false;
  if (nchunks == 1) {
    const PlanArgs pa = plan ? *plan : PlanArgs{nullptr, nullptr, 0, 0, 0};
    const int64_t nblocks = xq ? (int64_t)T * (d / BLK) : 0;  // no quantisation without xq
    const int64_t qblocks = (nblocks * 8 + PERM_CHUNK - 1) / PERM_CHUNK;
    hipLaunchKernelGGL(permute_small_kernel, dim3((unsigned)(1 + qblocks)), dim3(PERM_CHUNK), 0, s, idx, T, K, E,
                       counts, offsets, row_token, pair_row, x, nblocks, xq, xs, pa);
    if (planned) *planned = plan != nullptr;
    return hipGetLastError();
  }
  hipLaunchKernelGGL(count_kernel, dim3(nchunks), dim3(PERM_CHUNK), 0, s, idx, T, K, E, chunk_cnt);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(256), 0, s, chunk_cnt, nchunks, E, chunk_off, counts, offsets);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(scatter_kernel, dim3(nchunks), dim3(PERM_CHUNK), 0, s, idx, T, K, E, chunk_off, offsets,
                     row_token, pair_row);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  return xq ? launch_quant(x, T, d, xq, xs, s) : hipSuccess;
}

}  // namespace moe
