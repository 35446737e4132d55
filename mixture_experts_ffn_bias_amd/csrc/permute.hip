// Token counting and expert-contiguous order ("DeepSeek-V3.2-Exp · MoE update",
// moe-forward excerpt: a count of the selected experts, then for each expert
// the tokens that chose it in ascending token order), and the FP8 quantisation
// of x that the expert Linear layers consume.
//
// The order is built without atomics on global memory and without a host
// round trip: each 256-token chunk marks, per expert, which of its tokens
// chose it (a 256-bit mask in LDS); the popcount of the mask gives the chunk's
// count and, below a token's bit, that token's rank.  A single-workgroup scan
// turns chunk counts into per-chunk bases, so every (token, choice) pair gets
// its final row directly and the order is deterministic.
#include "permute_dev.h"

namespace moe {

namespace {

// grid = chunks, block = PERM_CHUNK
__global__ __launch_bounds__(PERM_CHUNK) void count_kernel(const int32_t* __restrict__ idx, int T, int K, int E,
                                                          int32_t* __restrict__ chunk_cnt) {
  __shared__ uint32_t mask[256 * MASK_WORDS];
  build_masks(mask, idx, T, K, E, blockIdx.x);
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
  build_masks(mask, idx, T, K, E, blockIdx.x);
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

// plan.tiles (may be NULL): also write the FFN tile list of one dense
// expert over the T rows (the MLP: tiles of plan.tile_rows rows, no routed
// experts), so that no plan kernel runs; T * d / 16 threads cover its
// ceil(T / tile_rows) entries.
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ x, int64_t nblocks,
                                                         uint8_t* __restrict__ q, float* __restrict__ scale,
                                                         PlanArgs plan, int T) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (plan.tiles) {
    const int nsh = (T + plan.tile_rows - 1) / plan.tile_rows;
    if (gid < nsh) st16<false>(plan.tiles + gid, shared_tile((int)gid, T, 0, plan.tile_rows, nsh, 0));
    if (gid == 0) *plan.n_tiles = nsh;
  }
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
  __shared__ PermLds L;
  permute_block(idx, T, K, E, counts, offsets, row_token, pair_row, plan, L);
}

}  // namespace

hipError_t launch_quant(const uint16_t* x, int64_t T, int d, uint8_t* xq, float* xs, hipStream_t s,
                        const PlanArgs* dense_plan) {
  const int64_t nblocks = T * (d / BLK);
  const int64_t threads = nblocks * 8;
  const PlanArgs pa = dense_plan ? *dense_plan : PlanArgs{nullptr, nullptr, 0, 0, 0};
  hipLaunchKernelGGL(quant_rows_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, x, nblocks, xq, xs,
                     pa, (int)T);
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
