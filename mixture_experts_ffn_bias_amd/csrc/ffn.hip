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
#include <algorithm>

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

// One item per workgroup.  UP: grid = max_tiles * items_per_tile(I/128, up_ks);
// down: grid = max_tiles * items_per_tile(ceil(d/256), dn_ks).  Block = 512.
// BF: bf16 weights and activations (64-element K blocks, no scales, h stored
// as bf16).  SPLIT: the instance for split K (kept apart so that the unsplit
// kernels carry none of its code).
template <bool UP, int ROWS, bool BF, bool SPLIT>
__global__ __launch_bounds__(512, 2 * Tile<ROWS>::OCC) void ffn_tiled_kernel(FfnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[Tile<ROWS>::template SMEM<BF>];
  Item<ROWS> it;
  if (!(UP ? up_item<ROWS, BF, SPLIT>(a, blockIdx.x, it) : down_item<ROWS, BF, SPLIT>(a, blockIdx.x, it)))
    return;  // uniform for the whole block, before any barrier
  ffn_run_item<UP, ROWS, BF, false, SPLIT>(a, it, smem);
}

// Stream-K up-projection of one dense expert (e4m3; FfnArgs::up_stream = L):
// workgroup b runs units [b L, b L + L) of tiles x h blocks x K blocks,
// segment by segment, each segment's partials into plane b - first(s).
// Grid: ceil(units / L).
template <int ROWS>
__global__ __launch_bounds__(512, 2 * Tile<ROWS>::OCC) void ffn_stream_up_kernel(FfnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[Tile<ROWS>::template SMEM<false>];
  const int nib = a.I / BLK, nkb = a.d / BLK, L = a.up_stream;
  const int64_t units = (int64_t)*a.n_tiles * nib * nkb;
  int64_t u = (int64_t)blockIdx.x * L;
  const int64_t u1 = min(u + L, units);
  while (u < u1) {  // uniform for the whole block
    const int s = (int)(u / nkb), kb0 = (int)(u - (int64_t)s * nkb);
    const int n = (int)min(u1 - u, (int64_t)(nkb - kb0));
    const int tile = s / nib;
    Item<ROWS> it;
    up_item_of<ROWS, false>(a, a.tiles[tile], s - tile * nib, it);
    item_krange<ROWS, false>(it, kb0, n, (int)blockIdx.x - stream_first(s, nkb, L));
    ffn_run_item<true, ROWS, false, false, true>(a, it, smem);
    u += n;
  }
}

// Split-K up-projection: g and u of each row summed over the slices in
// order, then what the unsplit epilogue does with them: h = bf16(silu(bf16 g)
// * bf16 u), the amax of each row's 128-column block, e4m3 h and its scale.
// 32 threads per (row, h block), 4 columns each; R * I / 4 threads in all
// (I a multiple of 128, so the 32 threads of a block are always all present).
// Stream-K (L > 0, one dense expert in tiles of NT rows, nkb K blocks):
// segment (tile, h block) s has stream_planes(s) planes instead of ks.
__global__ __launch_bounds__(256) void ffn_up_reduce_kernel(const float* __restrict__ part, int ks, int64_t R, int I,
                                                            int L, int nkb, int NT, uint8_t* __restrict__ hq,
                                                            float* __restrict__ hs) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // 4-column chunk
  const int nq = I / 4;
  if (i >= R * nq) return;
  const int64_t row = i / nq;
  const int c = (int)(i - row * nq) * 4;
  if (L > 0) ks = stream_planes((int)(row / NT) * (I / BLK) + c / BLK, nkb, L);
  const size_t plane = (size_t)R * 2 * I;
  const float* src = part + (size_t)row * 2 * I + c;
  float gs[4] = {0.f, 0.f, 0.f, 0.f}, us[4] = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < ks; ++k) {
    const float4 gv = *(const float4*)(src + k * plane), uv = *(const float4*)(src + k * plane + I);
    gs[0] += gv.x; gs[1] += gv.y; gs[2] += gv.z; gs[3] += gv.w;
    us[0] += uv.x; us[1] += uv.y; us[2] += uv.z; us[3] += uv.w;
  }
  float h[4], amax = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float gv = round_bf16(gs[j]), uv = round_bf16(us[j]);
    h[j] = round_bf16(gv / (1.f + expf(-gv)) * uv);
    amax = fmaxf(amax, fabsf(h[j]));
  }
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  const float sc = amax == 0.f ? 1.f : amax / E4M3_MAX;
  *(uint32_t*)(hq + row * I + c) = pack4_e4m3(h[0] / sc, h[1] / sc, h[2] / sc, h[3] / sc);
  if ((c & (BLK - 1)) == 0) hs[row * (I / BLK) + c / BLK] = sc;
}

// Split-K down-projection: out[r] = bf16(sum over slices k in order of
// part[k][r]), 8 features per thread.
__global__ __launch_bounds__(256) void ffn_reduce_kernel(const float* __restrict__ part, int ks, int64_t R, int d,
                                                         uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // 8-feature chunk
  if (i >= R * (d / 8)) return;
  const size_t plane = (size_t)R * d;
  float y[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) y[j] = 0.f;
  for (int k = 0; k < ks; ++k) {
    const float4 lo = *(const float4*)(part + k * plane + 8 * i), hi = *(const float4*)(part + k * plane + 8 * i + 4);
    y[0] += lo.x; y[1] += lo.y; y[2] += lo.z; y[3] += lo.w;
    y[4] += hi.x; y[5] += hi.y; y[6] += hi.z; y[7] += hi.w;
  }
  uint4 o;
  o.x = (uint32_t)f32_to_bf16(y[0]) | ((uint32_t)f32_to_bf16(y[1]) << 16);
  o.y = (uint32_t)f32_to_bf16(y[2]) | ((uint32_t)f32_to_bf16(y[3]) << 16);
  o.z = (uint32_t)f32_to_bf16(y[4]) | ((uint32_t)f32_to_bf16(y[5]) << 16);
  o.w = (uint32_t)f32_to_bf16(y[6]) | ((uint32_t)f32_to_bf16(y[7]) << 16);
  *(uint4*)(out + 8 * i) = o;
}

template <int ROWS, bool BF>
hipError_t launch_gemms(const FfnArgs& a, int64_t max_tiles, hipStream_t s, hipEvent_t* ev) {
  const int64_t R = (int64_t)a.T * a.K + a.T;
  // stream-K: one dense expert, ceil(T / ROWS) tiles, runs of up_stream units
  const int64_t g1 = a.up_stream > 0
                         ? ((int64_t)(a.T + ROWS - 1) / ROWS * (a.I / BLK) * (a.d / BLK) + a.up_stream - 1) / a.up_stream
                         : max_tiles * items_per_tile(a.I / BLK, a.up_ks);
  const int64_t g2 = max_tiles * items_per_tile((a.d / BLK + 1) / 2, a.dn_ks);
  record_event(ev, 0, s);
  if (!BF && a.up_stream > 0) {
    if constexpr (ROWS == 32)
      return hipErrorInvalidValue;  // the host picks stream-K for 64- and 128-row tiles only
    else
      hipLaunchKernelGGL(ffn_stream_up_kernel<ROWS>, dim3((unsigned)g1), dim3(512), 0, s, a);
  } else if (!BF && a.up_ks > 1) {
    hipLaunchKernelGGL((ffn_tiled_kernel<true, ROWS, false, true>), dim3((unsigned)g1), dim3(512), 0, s, a);
  } else {
    hipLaunchKernelGGL((ffn_tiled_kernel<true, ROWS, BF, false>), dim3((unsigned)g1), dim3(512), 0, s, a);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (!BF && (a.up_ks > 1 || a.up_stream > 0)) {
    const int64_t chunks = R * (a.I / 4);
    hipLaunchKernelGGL(ffn_up_reduce_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, s, a.part,
                       a.up_ks, R, a.I, a.up_stream, a.d / BLK, ROWS, a.hq, a.hs);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  record_event(ev, 1, s);
  if (!BF && a.dn_ks > 1)
    hipLaunchKernelGGL((ffn_tiled_kernel<false, ROWS, false, true>), dim3((unsigned)g2), dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL((ffn_tiled_kernel<false, ROWS, BF, false>), dim3((unsigned)g2), dim3(512), 0, s, a);
  err = hipGetLastError();
  if (err == hipSuccess && !BF && a.dn_ks > 1) {
    const int64_t chunks = R * (a.d / 8);
    hipLaunchKernelGGL(ffn_reduce_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, s, a.part, a.dn_ks,
                       R, a.d, a.out);
    err = hipGetLastError();
  }
  record_event(ev, 2, s);
  return err;
}

}  // namespace

int ffn_tile_rows(int64_t T, bool dense, bool bf16) {
  // A dense MLP of 33..128 rows streams the same weights for every tile:
  // 64-row tiles cut the workgroups that stream each weight byte to one or
  // two.  Routed experts with e4m3 weights: up to 768 tokens (experts of
  // about 24 rows on average) the weights are the traffic and narrow tiles
  // let two workgroups share a CU; then 64-row tiles (one workgroup per CU,
  // three stages) up to 1280, and 128-row tiles beyond (measured, whole
  // layer, ms: 512 tokens 2.22 with 128-row tiles / 1.89 with 32; 1024:
  // 2.41 / 2.34 / 2.26 with 64; 1536: 2.61 / 2.83 / 2.70).  With bf16
  // weights the 128-row tiles (three stages) are as fast or faster from 129
  // tokens on.
  if (dense) {
    if (T > 32 && T <= 128) return 64;
    return T <= 128 ? 32 : 128;
  }
  if (bf16) return T <= 128 ? 32 : 128;
  if (T <= 768) return 32;
  return T <= 1280 ? 64 : 128;
}

int64_t ffn_max_tiles(int64_t T, int K, int E, int tile_rows) {
  return (T * K) / tile_rows + E + (T + tile_rows - 1) / tile_rows + 1;
}

namespace {

// K slices of one projection: `items` items of nkb K blocks each, `slots`
// workgroups resident at once, pbytes of fp32 partials per slice.  Cost
// model, in units of one K block's time: the items run in rounds of `slots`,
// each taking its K blocks plus about two blocks of start-up and epilogue;
// the partial planes, written and read back, cost their bytes at the rate of
// one round's weight stream (slots x 32 KiB per block time).  A split is
// taken only when it beats the unsplit cost by 10 %.  Returns the cost of
// the choice.
double pick_ksplit(int64_t items, int nkb, int slots, double pbytes, int* ks, int* kper) {
  auto rounds = [&](int64_t n) { return (double)((n + slots - 1) / slots); };
  const double unsplit = rounds(items) * (nkb + 2);
  double best = unsplit * 0.9;
  *ks = 1;
  *kper = nkb;
  for (int k = 2; k <= 16; ++k) {
    const int per = (nkb + k - 1) / k;
    if (per < 4) break;
    const int kk = (nkb + per - 1) / per;  // no empty slice
    const double cost = rounds(items * kk) * (per + 2) + kk * 2.0 * pbytes / (slots * 32768.0);
    if (cost < best) {
      best = cost;
      *ks = kk;
      *kper = per;
    }
  }
  return *ks == 1 ? unsplit : best;
}

// Stream-K alternative, same units: `units` K blocks in runs of
// L = max(4, ceil(units / slots)), one run per workgroup; a run crosses up to
// ceil(L / nkb) + 1 segments (tile, block), each with its own start-up;
// *planes: the most runs that share one segment.
double stream_cost(int64_t units, int nkb, int slots, double pbytes, int* L, int* planes) {
  const int l = (int)std::max<int64_t>(4, (units + slots - 1) / slots);
  const int64_t runs = (units + l - 1) / l;
  int np = 1;
  for (int64_t sg = 0; sg < units / nkb; ++sg) np = std::max(np, stream_planes((int)sg, nkb, l));
  *L = l;
  *planes = np;
  const int segs = (l + nkb - 1) / nkb + 1;
  return (double)((runs + slots - 1) / slots) * (l + 2 * segs) + np * 2.0 * pbytes / (slots * 32768.0);
}

}  // namespace

void ffn_dense_ksplit(int64_t T, int d, int I, int* up_ks, int* up_kper, int* dn_ks, int* dn_kper, int* up_stream,
                      int* up_planes) {
  const int NT = ffn_tile_rows(T, true);
  const int slots = 256 * (NT == 32 ? Tile<32>::OCC : NT == 64 ? Tile<64>::OCC : Tile<128>::OCC);
  const int64_t tiles = (T + NT - 1) / NT;
  const double up_bytes = (double)T * 2 * I * 4;  // one plane of up-projection partials
  const double sliced = pick_ksplit(tiles * (I / BLK), d / BLK, slots, up_bytes, up_ks, up_kper);
  *up_planes = *up_ks > 1 ? *up_ks : 0;
  *up_stream = 0;
  int L = 0, np = 0;
  // stream-K only where it beats the best slicing by 5 % (and not with
  // 32-row tiles, whose single-row batches gain nothing from it)
  if (NT != 32 && stream_cost(tiles * (I / BLK) * (d / BLK), d / BLK, slots, up_bytes, &L, &np) < 0.95 * sliced) {
    *up_stream = L;
    *up_planes = np;
    *up_ks = 1;
    *up_kper = d / BLK;
  }
  pick_ksplit(tiles * ((d / BLK + 1) / 2), I / BLK, slots, (double)T * d * 4, dn_ks, dn_kper);
}

int ffn_plan_cap(int64_t T, int K, int E, bool has_shared, bool bf16) {
  const int NT = ffn_tile_rows(T, false, bf16);
  return (int)(ffn_max_tiles(T, K, E, NT) - (has_shared ? (T + NT - 1) / NT : 0));
}

hipError_t launch_ffn(const ExpertPtrs& routed, const ExpertPtrs* shared, int T, int d, int I, int E, int K,
                      const int32_t* offsets, const int32_t* row_token, const uint8_t* xq, const float* xs,
                      int4* tiles, int32_t* n_tiles, uint8_t* hq, float* hs, uint16_t* out, hipStream_t s,
                      hipEvent_t* ev, bool bf16, int e_lo, int e_hi, bool planned, const FfnSplit* split) {
  if (e_hi < 0) e_hi = E;
  const bool dense = K == 0;  // one dense expert (the MLP)
  const int NT = ffn_tile_rows(T, dense, bf16);
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
  a.part = split ? split->part : nullptr;
  a.up_ks = split && !bf16 ? split->up_ks : 1;  // split K: e4m3 only
  a.up_kper = split ? split->up_kper : 0;
  a.dn_ks = split && !bf16 ? split->dn_ks : 1;
  a.dn_kper = split ? split->dn_kper : 0;
  a.up_stream = split && !bf16 ? split->up_stream : 0;
  if (NT == 32) return bf16 ? launch_gemms<32, true>(a, max_tiles, s, ev) : launch_gemms<32, false>(a, max_tiles, s, ev);
  if (NT == 64) return bf16 ? hipErrorInvalidValue : launch_gemms<64, false>(a, max_tiles, s, ev);
  return bf16 ? launch_gemms<128, true>(a, max_tiles, s, ev) : launch_gemms<128, false>(a, max_tiles, s, ev);
}

}  // namespace moe
