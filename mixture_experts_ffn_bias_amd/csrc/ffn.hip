// Grouped SwiGLU expert FFN with FP8 (e4m3) weights and activations
// ("DeepSeek-V3.2-Exp · Gate projection": the expert excerpt, SwiGLU of the
// w1 and w3 projections taken in fp32, cast back to the input dtype, then w2;
// the Linear excerpt: FP8 weights [out, in] with one fp32 scale per 128x128
// block).
//
// Work unit ("tile"): up to 128 consecutive permuted rows of one expert.
// Up-projection workgroups own (tile, 128-column block of h) and hold the w1
// and w3 rows of that block, so the whole 128-wide block of h is in one
// workgroup, which applies SwiGLU and quantises h to e4m3 in its epilogue.
// Down-projection workgroups own (tile, 256 output features).
//
// Each 128-deep scale block is one block_dot (four bf16 MFMAs on exactly
// decoded e4m3 operands), so each block sum is scaled once:
// acc += P * (s_weight[block] * s_act[row, block]).
// Weights are the A operand (16 output features), activations the B operand
// (16 rows); lane l ends with features 4*(l/16)+j of row l%16.
#include "ffn_tile.h"
#include "plan.h"

namespace moe {

namespace {

// One block of 256 threads: the tile list from the expert offsets
// (plan_tiles_block).  The shared expert's tiles come first: they hold the
// most rows when T is small, and starting the longest work first keeps it
// off the end of the launch.
__global__ __launch_bounds__(256) void plan_tiles_kernel(const int32_t* __restrict__ offsets, int e_lo, int e_hi,
                                                         int T, int K, int NT, int has_shared, int cap,
                                                         int4* __restrict__ tiles, int32_t* __restrict__ n_tiles) {
  __shared__ int s[256];
  const int e = threadIdx.x;
  const int TK = T * K;
  int lo = 0, cnt = 0;
  if (e >= e_lo && e < e_hi) {
    lo = clampi(offsets[e], 0, TK);
    cnt = clampi(offsets[e + 1], lo, TK) - lo;
  }
  plan_tiles_block(lo, cnt, T, K, NT, has_shared, cap, e_lo, e_hi, s, tiles, n_tiles);
}

// One item per workgroup.  UP: grid = max_tiles * (I/128); down: grid =
// max_tiles * ceil(d/256).  Block = 512.  BF: bf16 weights and activations
// (64-element K blocks, no scales, h stored as bf16).
template <bool UP, int ROWS, bool BF>
__global__ __launch_bounds__(512, 2 * Tile<ROWS>::OCC) void ffn_tiled_kernel(FfnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[Tile<ROWS>::template SMEM<BF>];
  Item<ROWS> it;
  if (!(UP ? up_item<ROWS, BF>(a, blockIdx.x, it) : down_item<ROWS, BF>(a, blockIdx.x, it)))
    return;  // uniform for the whole block, before any barrier
  ffn_run_item<UP, ROWS, BF>(a, it, smem);
}

template <int ROWS, bool BF>
hipError_t launch_gemms(const FfnArgs& a, int64_t max_tiles, hipStream_t s, hipEvent_t* ev) {
  const int64_t g1 = max_tiles * (a.I / BLK);
  const int64_t g2 = max_tiles * ((a.d / BLK + 1) / 2);
  if (ev) (void)hipEventRecord(ev[0], s);
  hipLaunchKernelGGL((ffn_tiled_kernel<true, ROWS, BF>), dim3((unsigned)g1), dim3(512), 0, s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (ev) (void)hipEventRecord(ev[1], s);
  hipLaunchKernelGGL((ffn_tiled_kernel<false, ROWS, BF>), dim3((unsigned)g2), dim3(512), 0, s, a);
  err = hipGetLastError();
  if (ev) (void)hipEventRecord(ev[2], s);
  return err;
}

}  // namespace

int ffn_tile_rows(int64_t T) {
  // small batches: experts hold a few rows each and the weights are the
  // traffic; narrow tiles let two workgroups share a CU
  return T <= 128 ? 32 : 128;
}

int64_t ffn_max_tiles(int64_t T, int K, int E, int tile_rows) {
  return (T * K) / tile_rows + E + (T + tile_rows - 1) / tile_rows + 1;
}

int ffn_plan_cap(int64_t T, int K, int E, bool has_shared) {
  const int NT = ffn_tile_rows(T);
  return (int)(ffn_max_tiles(T, K, E, NT) - (has_shared ? (T + NT - 1) / NT : 0));
}

hipError_t launch_ffn(const ExpertPtrs& routed, const ExpertPtrs* shared, int T, int d, int I, int E, int K,
                      const int32_t* offsets, const int32_t* row_token, const uint8_t* xq, const float* xs,
                      int4* tiles, int32_t* n_tiles, uint8_t* hq, float* hs, uint16_t* out, hipStream_t s,
                      hipEvent_t* ev, bool bf16, int e_lo, int e_hi, bool planned) {
  if (e_hi < 0) e_hi = E;
  const int NT = ffn_tile_rows(T);
  const int64_t max_tiles = ffn_max_tiles(T, K, E, NT);
  const int nsh = shared ? (T + NT - 1) / NT : 0;
  if (!planned) {
    hipLaunchKernelGGL(plan_tiles_kernel, dim3(1), dim3(256), 0, s, offsets, e_lo, e_hi, T, K, NT, shared ? 1 : 0,
                       (int)(max_tiles - nsh), tiles, n_tiles);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  FfnArgs a;
  a.routed = routed;
  a.shared = shared ? *shared : routed;
  a.E = e_hi - e_lo;  // routed experts in `routed`; tiles of expert a.E are the shared expert's
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
  if (NT == 32) return bf16 ? launch_gemms<32, true>(a, max_tiles, s, ev) : launch_gemms<32, false>(a, max_tiles, s, ev);
  return bf16 ? launch_gemms<128, true>(a, max_tiles, s, ev) : launch_gemms<128, false>(a, max_tiles, s, ev);
}

}  // namespace moe
