// The FFN tile list, built by one 256-thread workgroup (kernels.h, launch_ffn:
// tiles[i] = {expert, first row, rows, (k << 1) | once}: k the tile's index
// within its expert, once = 1 for an expert's only tile).  Used by the plan kernel and,
// for small batches, by the single-launch permutation, which has the expert
// offsets at hand already.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace moe {

// Tile j of the shared expert (number e_sh, permuted rows [TK, TK + T), nsh
// tiles): NT rows each in row order, the last one ragged.
__device__ __forceinline__ uint4 shared_tile(int j, int T, int TK, int NT, int nsh, int e_sh) {
  return make_uint4(e_sh, TK + j * NT, min(NT, T - j * NT), (j << 1) | (nsh == 1 ? 1 : 0));
}

// Thread e (0..255) brings expert e's permuted rows [lo, lo + cnt) (ignored
// outside [e_lo, e_hi)); threads from 256 on only join the barriers.  s is
// 256 ints of LDS.  Routed experts [e_lo, e_hi)
// are numbered from e_lo; with has_shared the shared expert (number
// e_hi - e_lo, rows [T*K, T*K + T)) is planned first.  once = 1 marks the
// only tile of its expert.  An expert with more rows than one tile holds
// gets ceil(rows / NT) tiles of equal size (rounded up to 16 rows, the MFMA
// sub-tile): every tile then streams the same weights, and even sizes give
// each item the same share of multiply work to overlap with that stream.  At most cap routed tiles are written.  COH: the
// list is written with agent-coherent stores (common.h, ld / st).
template <bool COH = false>
__device__ __forceinline__ void plan_tiles_block(int lo, int cnt, int T, int K, int NT, int has_shared, int cap,
                                                 int e_lo, int e_hi, int* s, int4* __restrict__ tiles,
                                                 int32_t* __restrict__ n_tiles) {
  const int e = threadIdx.x;
  const bool act = e < 256;
  const int TK = T * K;
  const int nsh = has_shared ? (T + NT - 1) / NT : 0;
  for (int j = threadIdx.x; j < nsh; j += blockDim.x)
    st16<COH>(tiles + j, shared_tile(j, T, TK, NT, nsh, e_hi - e_lo));
  const int n = (act && e >= e_lo && e < e_hi) ? (cnt + NT - 1) / NT : 0;
  if (act) s[e] = n;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int v = act && e >= o ? s[e - o] : 0;
    __syncthreads();
    if (act) s[e] += v;
    __syncthreads();
  }
  const int base = act ? s[e] - n : 0;
  const int rt = n > 1 ? min(NT, ((cnt + n - 1) / n + 15) / 16 * 16) : NT;
  for (int j = 0; j < n && base + j < cap; ++j)
    st16<COH>(tiles + nsh + base + j, make_uint4(e - e_lo, lo + j * rt, min(rt, cnt - j * rt), (j << 1) | (n == 1 ? 1 : 0)));
  if (threadIdx.x == 0) st<COH>(n_tiles, (int32_t)(nsh + min(s[255], cap)));
}

}  // namespace moe
