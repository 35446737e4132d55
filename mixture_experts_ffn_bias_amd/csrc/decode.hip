// The whole MoE layer in one kernel launch for small batches (decode): router,
// permutation, expert FFN (routed and shared) and combine
// ("DeepSeek-V3.2-Exp · MoE update", moe-forward excerpt, every step of it;
// "DeepSeek-V3.2-Exp · Add shared output", formula).  The arithmetic is the
// same device code the per-step kernels run (gate_dev.h, permute_dev.h,
// ffn_tile.h, combine_dev.h); only the scheduling differs.
//
// Every workgroup runs one work item, chosen by its index.  Items are
// numbered so that each depends only on items with smaller numbers:
//   quantisation of x | router partial logits | shared-expert up-projection
//   | selection | permutation + tile list | routed up-projection
//   | down-projection (shared tiles first) | combine.
// The shared expert does not depend on the routing, so its up-projection
// streams its weights while the router and the permutation run, and a
// tile's down-projection starts as soon as that tile's up-projection is done
// rather than after the whole up-projection.
//
// Completion counts live in a control block at the start of the workspace.
// Everything one item hands to another is written with agent-coherent stores
// (common.h, ld / st: through to the memory all XCDs share), so no L2
// writeback or invalidation is needed (per workgroup, those cost the FFN a
// third of its bandwidth): a producer's waves wait until their stores have
// completed, then one thread bumps the count; a consumer's first thread polls
// it and the workgroup barrier releases the other threads, whose loads come
// after.  A consumer may read through its L2 (which holds nothing of the
// workspace at launch) because every cache line it reads is complete before
// any workgroup reads it, with one exception: a line of the FFN's activation
// scales spans rows of tiles that finish at different times, so those are
// copied with agent-coherent loads.  The waits
// are bounded: a workgroup that has polled too long marks the call as
// stalled and skips its work (the result is then garbage and the status
// word says so), so the launch always ends.  Since workgroups are handed out
// in index order within each dispatcher, an item only ever waits for items
// that are already running or done, and the bound is never reached.  The
// last workgroup to finish zeroes the counts for the next call and stores
// the call's status word.
#include "combine_dev.h"
#include "ffn_tile.h"
#include "gate_dev.h"
#include "kernels.h"
#include "permute_dev.h"

namespace moe {

namespace {

constexpr int DEC_THREADS = 512;
constexpr int DEC_ROWS = 32;                 // FFN tile rows
constexpr int DEC_SPIN_LIMIT = 1 << 21;      // polls before a wait gives up (far beyond any real wait)

struct DecodeArgs {
  FfnArgs f;  // E, d, I, T, K, experts, tile list, row_token, xq/xs, hq/hs, out (= the FFN output rows)
  const uint16_t* x;
  const float* gate_w;
  const float* gate_b;
  int G, TG;
  float route_scale;
  float* zpart;
  int32_t* idx;
  float* w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* pair_row;
  uint16_t* delta;
  int* ctl;
  int cap, max_tiles, nsh;
  int gate_kz, gate_kchunk, comb_parts;
  // first item of each range
  int b_gate, b_sup, b_sel, b_plan, b_rup, b_down, b_comb, b_end;
};

// Poll (thread 0) until ctl[i] >= target; then every thread may read what
// the counted items wrote.  False when the call has stalled.  The first look
// goes through the XCD's L2: a count only grows during a launch and the L2
// holds none at launch, so a cached value can only be short, never early;
// once a count is complete, the other workgroups of the XCD that wait for it
// see so without a round trip to memory.  Otherwise the count is polled
// with agent-coherent loads.
__device__ bool dec_wait(int* ctl, int i, int target, int* s_ok) {
  if (threadIdx.x == 0) {
    int ok = 1;
    if (__hip_atomic_load(ctl + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target)
    for (int n = 0;; ++n) {
      if (__hip_atomic_load(ctl + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) break;
      if (__hip_atomic_load(ctl + DEC_CTL_STALLED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0 ||
          n >= DEC_SPIN_LIMIT) {
        __hip_atomic_store(ctl + DEC_CTL_STALLED, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = 0;
        break;
      }
      if (n < 8)  // back off: long waits poll less
        __builtin_amdgcn_s_sleep(2);
      else
        __builtin_amdgcn_s_sleep(16);
    }
    *s_ok = ok;
  }
  __syncthreads();
  const bool ok = *s_ok != 0;
  __syncthreads();  // read by every thread before the next wait may rewrite it
  return ok;
}

// Count this workgroup's item as done: every wave's (agent-coherent) stores
// have completed before thread 0 bumps the count.
__device__ void dec_signal(int* ctl, int i) {
  asm volatile("" ::: "memory");  // no store moves below the wait
  wait_vmcnt<0>();
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(ctl + i, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Tile-list entry of the shared expert's tile j (as the plan writes it).
__device__ int4 shared_tile(const DecodeArgs& a, int j) {
  const FfnArgs& f = a.f;
  return make_int4(f.E, f.T * f.K + j * DEC_ROWS, min(DEC_ROWS, f.T - j * DEC_ROWS), (j << 1) | (a.nsh == 1 ? 1 : 0));
}

// The next item of a range from its counter (every workgroup of the range
// takes one, so the items handed out are exactly the range's).  Items taken
// this way still only wait for items of earlier ranges, all of whose
// workgroups each dispatcher starts before any of this range.  (Measured:
// worth it for the short down-projection items, where the XCDs' different
// rates leave a tail; not for the up-projection, whose tail the
// down-projection fills.)
__device__ int take_ticket(int* ctl, int i, int* s) {
  if (threadIdx.x == 0) *s = __hip_atomic_fetch_add(ctl + i, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int t = *s;
  __syncthreads();
  return t;
}

__device__ bool stalled(const int* ctl) {
  return __hip_atomic_load(ctl + DEC_CTL_STALLED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
}

__global__ __launch_bounds__(DEC_THREADS, 4) void decode_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[Tile<DEC_ROWS>::SMEM<false>];
  __shared__ int s_ok;
  const FfnArgs& f = a.f;
  const int b = blockIdx.x;
  const int T = f.T, E = f.E, d = f.d, K = f.K;
  const int nib = f.I / BLK, nob2 = (d / BLK + 1) >> 1;
  int* ctl = a.ctl;

  if (b < a.b_gate) {
    // quantisation of x: 64 blocks of 128 values per item, 8 lanes each
    const int64_t gid = (int64_t)b * DEC_THREADS + threadIdx.x;
    const int64_t blk = gid >> 3;
    if (blk < (int64_t)T * (d / BLK))
      quant_block<true>(a.x, blk, (int)(gid & 7), const_cast<uint8_t*>(f.xq), const_cast<float*>(f.xs));
    dec_signal(ctl, DEC_CTL_QUANT);
  } else if (b < a.b_sup) {
    // router partial logits: 16 experts x one K chunk, as two halves; wave
    // w: tokens 16 (w & 3) .. +16, half w >> 2
    const int g = b - a.b_gate;
    const int et = g / a.gate_kz, z = g - et * a.gate_kz;
    const int wave = threadIdx.x >> 6;
    const int t0 = 16 * (wave & 3), half = wave >> 2;
    const int hk = a.gate_kchunk / 2;
    const int k0 = min(d, z * a.gate_kchunk + half * hk), k1 = min(d, k0 + hk);
    if (t0 < T)
      gate_logits_wave<1, true>(a.x, a.gate_w, a.zpart + (size_t)(2 * z + half) * T * E, T, d, E, t0, 16 * et, 1, k0,
                             k1);
    dec_signal(ctl, DEC_CTL_GATE);
  } else if (b < a.b_sel) {
    // shared-expert up-projection: needs only the quantised x
    const int i = b - a.b_sup;
    const int j = i / nib;
    if (dec_wait(ctl, DEC_CTL_QUANT, a.b_gate, &s_ok)) {
      Item<DEC_ROWS> it;
      up_item_of<DEC_ROWS, false>(f, shared_tile(a, j), i - j * nib, it);
      ffn_run_item<true, DEC_ROWS, false, true>(f, it, smem);
    }
    dec_signal(ctl, DEC_CTL_UP + j);
  } else if (b < a.b_plan) {
    // selection: one token per wave
    const int nsel_tok = 8 * (b - a.b_sel) + (threadIdx.x >> 6);
    const int n_gate = a.b_sup - a.b_gate;
    if (dec_wait(ctl, DEC_CTL_GATE, n_gate, &s_ok)) {
      GateSlot* slots = reinterpret_cast<GateSlot*>(smem);
      GateSlot& sl = slots[threadIdx.x >> 6];
      const int tt = min(nsel_tok, T - 1);
      gate_scores_wave(a.zpart, 2 * a.gate_kz, a.gate_b, T, E, tt, sl);
      gate_choose_wave<true>(sl, E, a.G, a.TG, K, a.route_scale, nsel_tok, nsel_tok < T, a.idx, a.w);
    }
    dec_signal(ctl, DEC_CTL_SELECT);
  } else if (b < a.b_rup) {
    // permutation and tile list (one item)
    if (dec_wait(ctl, DEC_CTL_SELECT, a.b_plan - a.b_sel, &s_ok)) {
      const PlanArgs plan{const_cast<int4*>(f.tiles), const_cast<int32_t*>(f.n_tiles), DEC_ROWS, 1, a.cap};
      permute_block<true>(a.idx, T, K, E, a.counts, a.offsets, const_cast<int32_t*>(f.row_token), a.pair_row, plan,
                          *reinterpret_cast<PermLds*>(smem));  // (its few loads of idx are agent-coherent too)
      // Tiles past the end of the list count as up-projected (once the list
      // is in memory), so a down-projection item needs to wait for its own
      // tile's count only, and then finds out from the list whether it has
      // work.
      asm volatile("" ::: "memory");
      wait_vmcnt<0>();
      __syncthreads();
      for (int t = ld<true>(f.n_tiles) + threadIdx.x; t < a.max_tiles; t += DEC_THREADS)
        __hip_atomic_store(ctl + DEC_CTL_UP + t, nib, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    dec_signal(ctl, DEC_CTL_PLAN);
  } else if (b < a.b_down) {
    // routed up-projection: tiles nsh.. of the list
    const int r = b - a.b_rup;
    const int tile = a.nsh + r / nib;
    if (dec_wait(ctl, DEC_CTL_PLAN, 1, &s_ok) && tile < *f.n_tiles) {
      Item<DEC_ROWS> it;
      up_item_of<DEC_ROWS, false>(f, f.tiles[tile], r - (r / nib) * nib, it);
      ffn_run_item<true, DEC_ROWS, false, true>(f, it, smem);
      dec_signal(ctl, DEC_CTL_UP + tile);
    }
  } else if (b < a.b_comb) {
    // down-projection of tile dn / nob2 once its up-projection is complete
    // (for a routed tile that also means the tile list is in memory; a
    // shared tile's entry is known without it)
    // The item is taken from a counter rather than from the workgroup index:
    // the XCDs (each gets every eighth workgroup) stream at different rates,
    // and the faster ones then take more of the items.
    const int dn = take_ticket(ctl, DEC_CTL_DTICKET, &s_ok);
    const int tile = dn / nob2;
    if (dec_wait(ctl, DEC_CTL_UP + tile, nib, &s_ok)) {
      const bool sh = tile < a.nsh;
      if (sh || tile < *f.n_tiles) {
        Item<DEC_ROWS> it;
        down_item_of<DEC_ROWS, false>(f, sh ? shared_tile(a, tile) : f.tiles[tile], dn - tile * nob2, it);
        ffn_run_item<false, DEC_ROWS, false, true>(f, it, smem);
        dec_signal(ctl, DEC_CTL_DOWN);
      }
    }
  } else {
    // combine: token c / parts, share c % parts of its row, after every down item
    const int c = b - a.b_comb;
    const int t = c / a.comb_parts;
    if (dec_wait(ctl, DEC_CTL_PLAN, 1, &s_ok)) {
      const int n_down = *f.n_tiles * nob2;
      if (dec_wait(ctl, DEC_CTL_DOWN, n_down, &s_ok))
        combine_token<false>(a.idx, a.w, a.pair_row, f.out, 1, T, K, 0, E, d, a.delta, t, c - t * a.comb_parts,
                             a.comb_parts, *reinterpret_cast<CombineLds*>(smem));
    }
  }

  // the last workgroup out resets the counts and stores the status
  __syncthreads();
  if (threadIdx.x == 0) {
    const int done = __hip_atomic_fetch_add(ctl + DEC_CTL_FINISHED, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == (int)gridDim.x - 1) {
      const int st = stalled(ctl) ? 1 : 0;
      for (int i = 0; i < DEC_CTL_UP; i += 32)
        if (i != DEC_CTL_STATUS) __hip_atomic_store(ctl + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int i = DEC_CTL_UP; i < DEC_CTL_UP + a.max_tiles; ++i)
        __hip_atomic_store(ctl + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(ctl + DEC_CTL_STATUS, st, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace

DecodeShape decode_shape(int T, int d, int I, int E, int K) {
  DecodeShape sh;
  sh.max_tiles = (int)ffn_max_tiles(T, K, E, DEC_ROWS);
  sh.nsh = (T + DEC_ROWS - 1) / DEC_ROWS;
  const int k64 = d / 64;  // router K in 64-wide steps (two 32-wide halves)
  sh.gate_kz = k64 < 8 ? k64 : 8;
  sh.gate_kchunk = ((k64 + sh.gate_kz - 1) / sh.gate_kz) * 64;
  sh.comb_parts = (d / 8 + DEC_THREADS - 1) / DEC_THREADS;
  const int nib = I / BLK, nob2 = (d / BLK + 1) / 2;
  const int64_t qthreads = (int64_t)T * (d / BLK) * 8;
  int b = (int)((qthreads + DEC_THREADS - 1) / DEC_THREADS);
  sh.b_gate = b;
  b += (E / 16) * sh.gate_kz;
  sh.b_sup = b;
  b += sh.nsh * nib;
  sh.b_sel = b;
  b += (T + 7) / 8;
  sh.b_plan = b;
  b += 1;
  sh.b_rup = b;
  b += (sh.max_tiles - sh.nsh) * nib;
  sh.b_down = b;
  b += sh.max_tiles * nob2;
  sh.b_comb = b;
  b += T * sh.comb_parts;
  sh.b_end = b;
  return sh;
}

hipError_t launch_decode(const DecodeShape& sh, const ExpertPtrs& routed, const ExpertPtrs& shared,
                         const uint16_t* x, const float* gate_w, const float* gate_b, int T, int d, int I, int E,
                         int G, int TG, int K, float route_scale, const DecodeBufs& bu, uint16_t* delta,
                         hipStream_t s) {
  DecodeArgs a;
  a.f = FfnArgs{routed, shared, E, d, I, T, K, bu.tiles, bu.n_tiles, bu.row_token, bu.xq, bu.xs, bu.hq, bu.hs,
                bu.rows};
  a.x = x;
  a.gate_w = gate_w;
  a.gate_b = gate_b;
  a.G = G;
  a.TG = TG;
  a.route_scale = route_scale;
  a.zpart = bu.zpart;
  a.idx = bu.idx;
  a.w = bu.w;
  a.counts = bu.counts;
  a.offsets = bu.offsets;
  a.pair_row = bu.pair_row;
  a.delta = delta;
  a.ctl = bu.ctl;
  a.cap = ffn_plan_cap(T, K, E, true);
  a.max_tiles = sh.max_tiles;
  a.nsh = sh.nsh;
  a.gate_kz = sh.gate_kz;
  a.gate_kchunk = sh.gate_kchunk;
  a.comb_parts = sh.comb_parts;
  a.b_gate = sh.b_gate;
  a.b_sup = sh.b_sup;
  a.b_sel = sh.b_sel;
  a.b_plan = sh.b_plan;
  a.b_rup = sh.b_rup;
  a.b_down = sh.b_down;
  a.b_comb = sh.b_comb;
  a.b_end = sh.b_end;
  hipLaunchKernelGGL(decode_kernel, dim3((unsigned)sh.b_end), dim3(DEC_THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
