// LDS-tiled work items of the SwiGLU expert FFN with e4m3 (or bf16) weights
// ("DeepSeek-V3.2-Exp · Gate projection": expert excerpt and the FP8 Linear
// with one fp32 scale per 128x128 weight block).  Shared by the grouped FFN
// kernels and the single-launch layer kernel: a work item is one tile of
// permuted rows of one expert and one block of output columns, run by one
// 512-thread workgroup through a global -> LDS copy pipeline.
#pragma once
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// token of permuted row `row` (NULL map: rows are tokens, as for a dense
// MLP).  Rows from TK = T*K on are the shared expert's, one per token in
// token order, so they need no lookup.
__device__ __forceinline__ int token_of(const int32_t* row_token, int row, int T, int TK) {
  if (!row_token) return row;
  return row >= TK ? min(row - TK, T - 1) : clampi(row_token[row], 0, T - 1);
}

// With e4m3 weights, xq/hq are e4m3 rows with block scales xs/hs; with bf16
// weights (no scales), xq is the bf16 input x, hq receives bf16 h and the
// scale pointers are unused.
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
  // Split K (a projection with too few items to occupy the chip): with
  // up_ks / dn_ks > 1, item (tile, block, slice k) of that projection
  // multiplies K blocks [k kper, k kper + kper) and stores fp32 partial rows
  // in part[k][row][...] (rows T*K + T): up: [2 I], g then u; down: [d].
  // The reduce kernels add the slices in order.
  float* part;
  int dn_ks, dn_kper;
  int up_ks, up_kper;
  // Stream-K up-projection of one dense expert (up_stream = L > 0): the
  // tiles x h blocks x K blocks units, in that order, are dealt in runs of L
  // to the workgroups; a run covers one or more (tile, h block) segments,
  // and workgroup b stores its part of segment s in partial plane
  // b - first(s), first(s) = s nkb / L (stream_first).
  int up_stream;
};

__host__ __device__ inline int stream_first(int s, int nkb, int L) { return (int)((int64_t)s * nkb / L); }
__host__ __device__ inline int stream_planes(int s, int nkb, int L) {
  return (int)(((int64_t)(s + 1) * nkb - 1) / L) - stream_first(s, nkb, L) + 1;
}

// Items of one tile in a projection of nblk blocks: with split K (ks > 1) the
// ks slices of a block are consecutive and the count is padded to a multiple
// of 8, so that the items of the tiles of one expert, which read the same
// weights, fall on the same XCD (workgroups are dealt to the eight XCDs in
// turn) and share its L2.
__host__ __device__ inline int items_per_tile(int nblk, int ks) { return ks > 1 ? (nblk * ks + 7) & ~7 : nblk; }

// ---------------------------------------------------------------------------
// LDS-tiled kernels.  A workgroup (8 waves) owns one tile of up to 128 rows
// and 256 weight rows in two groups of 128:
//   up-projection:   group 0 = w1 rows of one 128-wide h block, group 1 = the
//                    w3 rows of the same block (so g and u of an h column meet
//                    in the same lane and the epilogue fuses SwiGLU + h quant);
//   down-projection: two consecutive 128-feature blocks of w2.
// Per 128-deep K block, the e4m3 weight (256 x 128 B) and activation
// (128 x 128 B) tiles and the activation scales are copied global -> LDS
// directly (global_load_lds, no register staging) into one of the NSTAGE
// stage buffers (Tile below), NSTAGE - 1 K blocks ahead of the multiply.
// Rows are stored unpadded with their 16-byte chunks XOR-permuted (swz),
// which makes the MFMA-layout reads bank-conflict free.  Wave (wr, wc)
// multiplies rows [64 wr, 64 wr + 64) by weight rows {32 wc .. 32 wc + 31}
// of both groups: 4 x 4 block products per K block.
// The weight copies of a tile that is the only one of its expert (at decode
// sizes, nearly every routed expert's) carry the non-temporal hint: those
// bytes are read exactly once, and full-line DMA streams with the hint reach
// a markedly higher HBM read rate on gfx950 (about 7.0 against 6.2 TB/s in a
// plain read test).
// Weights that other tiles read again are loaded with the default policy so
// that the L2 can serve the repeat reads.
// ---------------------------------------------------------------------------

constexpr int TT_WROWS = 256;                // weight rows per tile
constexpr int TT_A_BYTES = TT_WROWS * BLK;   // one K block of the weight tile
constexpr int CPOL_NT = 2;                   // cache-policy bits of a non-temporal load (gfx94x/gfx950)
constexpr int CPOL_SC1 = 16;                 // ... of an agent-coherent load (common.h, ld / st)

// Shape of the LDS pipeline for tiles of ROWS activation rows.  A stage holds
// one K block: the 256 weight rows, the ROWS activation rows and their scales.
// NSTAGE<BF> stages: the copies of NSTAGE - 1 K blocks are in flight while
// one is multiplied.
//   ROWS = 128, one workgroup per CU (its registers allow no more): two
//     stages (97 KiB) with e4m3 weights, where a third measured 3-4 % slower
//     on every large batch; three (146 KiB) with bf16 weights, which carry
//     twice the bytes and no decode work and measured 12 % faster with the
//     third.
//   ROWS = 32 (small batches, where the weights are the traffic): two stages
//     of 36 KiB and at most 128 VGPRs, so two workgroups share a CU and one's
//     start-up and epilogue overlap the other's weight stream.
//   ROWS = 64 (a dense MLP of 33..128 rows): one workgroup per CU with three
//     stages (121 KiB), so two K blocks of weights are in flight per CU and
//     each weight byte is streamed by at most two workgroups; only the
//     first row of waves multiplies (as with 32 rows).
template <int ROWS>
struct Tile {
  static_assert(ROWS == 32 || ROWS == 64 || ROWS == 128, "tile rows");
  static constexpr int B_BYTES = ROWS * BLK;
  static constexpr int S_BYTES = ROWS * 4;
  static constexpr int STAGE = TT_A_BYTES + B_BYTES + S_BYTES;
  template <bool BF>
  static constexpr int NSTAGE = ROWS == 64 || (ROWS == 128 && BF) ? 3 : 2;
  template <bool BF>
  static constexpr int SMEM = NSTAGE<BF> * STAGE;
  static constexpr int OCC = ROWS == 32 ? 2 : 1;        // workgroups per CU (8 waves each: 2 OCC waves per SIMD)
  static constexpr int APW = ROWS == 128 ? 2 : 1;       // 8-row activation pieces per copying wave
  static constexpr int AWAVES = ROWS / (8 * APW);       // waves that copy activation rows
  static constexpr int SWAVES = (ROWS + 63) / 64;       // waves that copy activation scales (64 rows each)
  static constexpr int MVMAX = ROWS >= 64 ? 4 : ROWS / 16;  // 16-row sub-tiles per wave
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* gbl_ptr_t;
// Read-only data addressed uniformly by the workgroup (the weight block
// scales): loads through the constant address space become scalar loads,
// which are counted apart from the vector-memory copies the pipeline waits on.
typedef const __attribute__((address_space(4))) float* const_f32_ptr;

// LDS holds each 128-byte row unpadded with its 16-byte chunks permuted:
// chunk c of row r sits at slot c ^ swz(r).  Sixteen consecutive rows then
// spread one MFMA-layout read (same chunk, rows r0..r0+15) over all banks.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// Wait until at most N of this wave's vector-memory operations are pending.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Global -> LDS copies (global_load_lds) of one K block.  Wave w copies
// weight rows [32w, 32w + 32) (four 8-row pieces), the APW 8-row activation
// pieces [APW w, APW w + APW) (waves w < AWAVES) and, e4m3 only, for
// w < SWAVES the scales of activation rows [64w, 64w + 64).  Lane l of a
// piece covers row piece_row0 + l/8 and LDS slot l%8, so it fetches global
// chunk (l%8) ^ swz(row).  WPOL / SPOL: cache policy of the weight and of the
// activation-scale copies.
template <int ROWS>
struct TileSrc {
  const uint8_t* a[4];                // this lane's source rows for the four weight pieces (chunk applied)
  const uint8_t* b[Tile<ROWS>::APW];  // ... for this wave's activation pieces
  const float* s;                     // scale row of activation row 64w + lane (waves w < SWAVES)
};

// act (wave-uniform): this wave's activation pieces hold rows some MFMA
// reads; otherwise they are not copied.
template <int ROWS, bool BF>
__device__ __forceinline__ int tile_copies(int wave, bool act) {
  using G = Tile<ROWS>;
  return 4 + (act ? G::APW : 0) + (!BF && wave < G::SWAVES ? 1 : 0);
}

template <int ROWS, bool BF, int WPOL, int SPOL>
__device__ __forceinline__ void tile_issue(const TileSrc<ROWS>& src, uint8_t* stage, int kb, int wave, bool act) {
  using G = Tile<ROWS>;
  const int off = kb * BLK;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    __builtin_amdgcn_global_load_lds((gbl_ptr_t)(src.a[i] + off), (lds_ptr_t)(stage + (wave * 4 + i) * 1024), 16, 0,
                                     WPOL);
  if (act) {
#pragma unroll
    for (int j = 0; j < G::APW; ++j)
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(src.b[j] + off),
                                       (lds_ptr_t)(stage + TT_A_BYTES + (wave * G::APW + j) * 1024), 16, 0, 0);
  }
  if (!BF && wave < G::SWAVES) {
    if (ROWS >= 64 || (threadIdx.x & 63) < ROWS)
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(src.s + kb),
                                       (lds_ptr_t)(stage + TT_A_BYTES + G::B_BYTES + wave * 256), 4, 0, SPOL);
  }
}

// Wait until at most n of this wave's vector-memory operations are pending
// (n wave-uniform, 0 <= n <= 14; larger values wait for all).
__device__ __forceinline__ void wait_vmcnt_upto(int n) {
  switch (__builtin_amdgcn_readfirstlane(n)) {
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 10: wait_vmcnt<10>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 14: wait_vmcnt<14>(); break;
    default: wait_vmcnt<0>(); break;
  }
}

// Workgroup barrier of the copy pipeline.  Each wave has already waited
// (wait_vmcnt) for its own global->LDS copies of the stage the barrier
// publishes, and the pipeline writes LDS in no other way, so no memory fence
// is needed: the fence __syncthreads adds would also wait for the copies of
// the stage after it.  The empty asm statements keep the compiler from moving
// LDS accesses across the barrier.
__device__ __forceinline__ void pipeline_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ v8i lds_frag(const uint8_t* base, int r, int g) {
  const uint8_t* row = base + r * BLK;
  const int z = swz(r);
  const v4i lo = *(const v4i*)(row + 16 * (g ^ z));
  const v4i hi = *(const v4i*)(row + 16 * ((4 + g) ^ z));
  return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// One K block of the tile: this wave's block products from the stage buffer
// `stage`, scaled and added to acc (MV: the wave's 16-row sub-tiles that hold
// rows; 0 multiplies nothing).
template <int ROWS, bool BF, int MV>
__device__ __forceinline__ void kblock_multiply(const uint8_t* stage, const_f32_ptr sa0, const_f32_ptr sa1, int kb,
                                                v4f (&acc)[2][2][Tile<ROWS>::MVMAX]) {
  using G = Tile<ROWS>;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  const int wr = wave >> 2, wc = wave & 3;
  if constexpr (BF && MV > 0) {
    // bf16 operands: the 128 bytes of a row are 64 k values, two MFMAs per block, no scales
    const uint8_t* la = stage;
    const uint8_t* lb = la + TT_A_BYTES;
    FragH B[MV];
#pragma unroll
    for (int m = 0; m < MV; ++m) B[m] = as_bf16(lds_frag(lb, wr * 64 + 16 * m + r, g));
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
        const FragH A = as_bf16(lds_frag(la, gi * 128 + wc * 32 + jt * 16 + r, g));
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int m = 0; m < MV; ++m)
            acc[gi][jt][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A.k[q], B[m].k[q], acc[gi][jt][m], 0, 0, 0);
      }
    }
  }
  if constexpr (!BF && MV > 0) {
    const uint8_t* la = stage;
    const uint8_t* lb = la + TT_A_BYTES;
    const float* ls = (const float*)(lb + G::B_BYTES);
    const float s_a0 = sa0[kb], s_a1 = sa1[kb];
    Frag B[MV];
    float sb[MV];
#pragma unroll
    for (int m = 0; m < MV; ++m) {
      B[m] = decode_e4m3(lds_frag(lb, wr * 64 + 16 * m + r, g));
      sb[m] = ls[wr * 64 + 16 * m + r];
    }
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
        const Frag A = decode_e4m3(lds_frag(la, gi * 128 + wc * 32 + jt * 16 + r, g));
        const float sg = gi == 0 ? s_a0 : s_a1;
        // MV independent accumulation chains, issued round-robin
        v4f p[MV];
#pragma unroll
        for (int m = 0; m < MV; ++m) p[m] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int m = 0; m < MV; ++m) p[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A.k[q], B[m].k[q], p[m], 0, 0, 0);
#pragma unroll
        for (int m = 0; m < MV; ++m) {
          const float f = sg * sb[m];
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[gi][jt][m][j] = fmaf(p[m][j], f, acc[gi][jt][m][j]);
        }
      }
    }
  }
}

// Main loop shared by both projections.  src: this lane's DMA sources.
// sa0, sa1: weight block scales of the two weight groups over K.
// acc[gi][jt][m].  MV: the 16-row sub-tiles of this wave that hold rows
// (0..4; a compile-time count keeps the K-block body free of branches, so the
// LDS reads, decodes and MFMAs of a block can be interleaved).  WPOL: cache
// policy of the weight copies.
template <int ROWS, bool BF, int MV, int WPOL, int SPOL>
__device__ __forceinline__ void tiled_mainloop(uint8_t* smem, const TileSrc<ROWS>& src, const_f32_ptr sa0,
                                               const_f32_ptr sa1, int nkb, int nrows,
                                               v4f (&acc)[2][2][Tile<ROWS>::MVMAX]) {
  using G = Tile<ROWS>;
  constexpr int NS = G::template NSTAGE<BF>;
  constexpr int AHEAD = NS - 1;  // K blocks whose copies are in flight during a multiply
  // scalar wave index: the LDS addresses of the copies are computed with scalar instructions
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  const bool act = wave < G::AWAVES && 16 * ((wave * G::APW * 8) >> 4) < nrows;
  const int per_stage = tile_copies<ROWS, BF>(wave, act);
  int issued = 0;
#pragma unroll
  for (int k = 0; k < AHEAD; ++k) {
    if (k < nkb) {
      tile_issue<ROWS, BF, WPOL, SPOL>(src, smem + k * G::STAGE, k, wave, act);
      ++issued;
    }
  }
  wait_vmcnt_upto(per_stage * (issued - 1));
  pipeline_barrier();

  // Iteration kb issues the copies of block kb + AHEAD into the stage that
  // block kb - 1 used (every wave left it at the last barrier), multiplies
  // block kb, then waits for its own copies of block kb + 1 (all but those of
  // the blocks issued after it); the barrier publishes that stage.
  auto step = [&](int cur, int kb) {  // cur = kb % NS
    const int nb = cur == 0 ? NS - 1 : cur - 1;  // (kb + AHEAD) % NS
    if (kb + AHEAD < nkb) tile_issue<ROWS, BF, WPOL, SPOL>(src, smem + nb * G::STAGE, kb + AHEAD, wave, act);
    // a wave whose 64 rows hold no tile row (MV = 0) only helps with the copies
    kblock_multiply<ROWS, BF, MV>(smem + cur * G::STAGE, sa0, sa1, kb, acc);
    if (kb + 1 < nkb) wait_vmcnt_upto(per_stage * (min(kb + AHEAD, nkb - 1) - kb - 1));
    pipeline_barrier();
  };
  if constexpr (ROWS == 128) {
    // unrolled over the NS stages: each stage's LDS offsets are constants, so
    // the addresses need no per-block arithmetic (prefill -2 %; the 32-row
    // kernels would spill)
    for (int kb = 0; kb < nkb; kb += NS) {
      step(0, kb);
      if (kb + 1 < nkb) step(1, kb + 1);
      if constexpr (NS == 3) {
        if (kb + 2 < nkb) step(2, kb + 2);
      }
    }
  } else {
    int cur = 0;
    for (int kb = 0; kb < nkb; ++kb) {
      step(cur, kb);
      cur = cur == NS - 1 ? 0 : cur + 1;
    }
  }
}

template <int ROWS, bool BF, int WPOL, int SPOL>
__device__ __forceinline__ void run_mainloop_pol(uint8_t* smem, const TileSrc<ROWS>& src, const_f32_ptr c0,
                                                 const_f32_ptr c1, int nkb, int nrows, int mvalid,
                                                 v4f (&acc)[2][2][Tile<ROWS>::MVMAX]) {
  if constexpr (Tile<ROWS>::MVMAX == 4) {
    switch (mvalid) {
      case 0: tiled_mainloop<ROWS, BF, 0, WPOL, SPOL>(smem, src, c0, c1, nkb, nrows, acc); break;
      case 1: tiled_mainloop<ROWS, BF, 1, WPOL, SPOL>(smem, src, c0, c1, nkb, nrows, acc); break;
      case 2: tiled_mainloop<ROWS, BF, 2, WPOL, SPOL>(smem, src, c0, c1, nkb, nrows, acc); break;
      case 3: tiled_mainloop<ROWS, BF, 3, WPOL, SPOL>(smem, src, c0, c1, nkb, nrows, acc); break;
      default: tiled_mainloop<ROWS, BF, 4, WPOL, SPOL>(smem, src, c0, c1, nkb, nrows, acc); break;
    }
  } else {
    switch (mvalid) {
      case 0: tiled_mainloop<ROWS, BF, 0, WPOL, SPOL>(smem, src, c0, c1, nkb, nrows, acc); break;
      case 1: tiled_mainloop<ROWS, BF, 1, WPOL, SPOL>(smem, src, c0, c1, nkb, nrows, acc); break;
      default: tiled_mainloop<ROWS, BF, 2, WPOL, SPOL>(smem, src, c0, c1, nkb, nrows, acc); break;
    }
  }
}

// The main loop for this tile (mvalid: wave-uniform count of this wave's
// 16-row sub-tiles that hold rows), with non-temporal weight copies when the
// tile reads them once.
template <int ROWS, bool BF, int SPOL>
__device__ __forceinline__ void run_mainloop(uint8_t* smem, const TileSrc<ROWS>& src, const float* sa0,
                                             const float* sa1, int nkb, int nrows, int mvalid, bool once,
                                             v4f (&acc)[2][2][Tile<ROWS>::MVMAX]) {
  const const_f32_ptr c0 = (const_f32_ptr)sa0, c1 = (const_f32_ptr)sa1;
  if (once)
    run_mainloop_pol<ROWS, BF, CPOL_NT, SPOL>(smem, src, c0, c1, nkb, nrows, mvalid, acc);
  else
    run_mainloop_pol<ROWS, BF, 0, SPOL>(smem, src, c0, c1, nkb, nrows, mvalid, acc);
}

// DMA source pointers of this lane.  wrow(i): weight row of tile row i
// (0..255); arow(j): activation row pointer of tile row j (0..127);
// srow(j): its scale row.
template <int ROWS, typename WRow, typename ARow, typename SRow>
__device__ __forceinline__ TileSrc<ROWS> make_tile_src(WRow wrow, ARow arow, SRow srow) {
  using G = Tile<ROWS>;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int slot = lane & 7;
  TileSrc<ROWS> t;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (wave * 4 + i) * 8 + (lane >> 3);
    t.a[i] = wrow(row) + 16 * (slot ^ swz(row));
  }
#pragma unroll
  for (int j = 0; j < G::APW; ++j) {
    const int row = min((wave * G::APW + j) * 8 + (lane >> 3), ROWS - 1);
    t.b[j] = arow(row) + 16 * (slot ^ swz(row));
  }
  t.s = srow(min(min(wave, G::SWAVES - 1) * 64 + lane, ROWS - 1));
  return t;
}

// LDS exchange barrier: this wave's LDS stores are complete (lgkmcnt) and
// every wave has arrived.  Unlike __syncthreads it does not wait for the
// wave's global -> LDS copies, which may still be in flight for the next
// K block.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One work item of a projection: a tile and a block of output columns.
template <int ROWS>
struct Item {
  TileSrc<ROWS> src;   // this lane's copy sources
  const float* sa0;    // weight block scales of the two weight groups over K (e4m3)
  const float* sa1;
  int blk;             // up: the 128-wide h block; down: the pair of 128-feature output blocks
  int expert;          // the tile's expert (routed experts first, then the shared one)
  int row0, nrows;     // the tile's permuted rows
  bool once;           // the tile is the only one of its expert
  int nkb;             // K blocks multiplied
  int kslice;          // K slice (split K), else 0
};

// Restrict an item to K blocks [kb0, kb0 + n) (n >= 1), its partials going
// to plane `plane`.
template <int ROWS, bool BF>
__device__ __forceinline__ void item_krange(Item<ROWS>& it, int kb0, int n, int plane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) it.src.a[i] += kb0 * BLK;
#pragma unroll
  for (int j = 0; j < Tile<ROWS>::APW; ++j) it.src.b[j] += kb0 * BLK;
  if (!BF) {
    it.src.s += kb0;
    it.sa0 += kb0;
    it.sa1 += kb0;
  }
  it.nkb = n;
  it.kslice = plane;
}

// Restrict an item to K slice k (K blocks [k kper, k kper + kper); the host
// picks the slicing so that no slice is empty).
template <int ROWS, bool BF>
__device__ __forceinline__ void item_kslice(Item<ROWS>& it, int k, int kper) {
  const int kb0 = k * kper;
  item_krange<ROWS, BF>(it, kb0, min(kper, it.nkb - kb0), k);
}

// Up-projection item of tile td (tile list entry: expert, first row, rows,
// once) and h block ib.
template <int ROWS, bool BF>
__device__ __forceinline__ void up_item_of(const FfnArgs& a, int4 td, int ib, Item<ROWS>& it) {
  constexpr int EB = BF ? 2 : 1;
  const int nib = a.I / BLK, nkb = a.d * EB / BLK;
  const int TK = a.T * a.K;
  const int e = td.x, row0 = td.y, nrows = td.z;
  const bool sh = e >= a.E;
  const ExpertPtrs& P = sh ? a.shared : a.routed;
  const size_t eo = sh ? 0 : (size_t)e;
  const int* rt = a.row_token;
  it.src = make_tile_src<ROWS>(
      [&](int row) {  // 0..127: w1 rows of block ib, 128..255: w3 rows
        const uint8_t* base = row < 128 ? P.w1 : P.w3;
        return base + (eo * a.I + ib * BLK + (row & 127)) * (size_t)a.d * EB;
      },
      [&](int row) {
        const int tok = token_of(rt, row0 + min(row, nrows - 1), a.T, TK);
        return a.xq + (size_t)tok * a.d * EB;
      },
      [&](int row) -> const float* {
        if (BF) return nullptr;
        const int tok = token_of(rt, row0 + min(row, nrows - 1), a.T, TK);
        return a.xs + (size_t)tok * nkb;
      });
  it.sa0 = BF ? nullptr : P.s1 + (eo * nib + ib) * nkb;
  it.sa1 = BF ? nullptr : P.s3 + (eo * nib + ib) * nkb;
  it.blk = ib;
  it.expert = e;
  it.row0 = row0;
  it.nrows = nrows;
  it.once = (td.w & 1) != 0;
  it.nkb = nkb;
  it.kslice = 0;
}

// Item `item` of the up-projection (tile item / nib, h block item % nib;
// with split K, tile item / items_per_tile, then h block and K slice); false
// past the last tile and for padding items.  SPLIT: the kernel instance that
// handles split K (a.up_ks is read only there).
template <int ROWS, bool BF, bool SPLIT>
__device__ __forceinline__ bool up_item(const FfnArgs& a, int item, Item<ROWS>& it) {
  const int nib = a.I / BLK;
  const int ks = SPLIT && a.up_ks > 1 ? a.up_ks : 1;
  const int per_tile = items_per_tile(nib, ks);
  const int tile = item / per_tile;
  const int rem = item - tile * per_tile;
  if (tile >= *a.n_tiles || rem >= nib * ks) return false;
  const int ib = rem / ks;
  up_item_of<ROWS, BF>(a, a.tiles[tile], ib, it);
  if (ks > 1) item_kslice<ROWS, BF>(it, rem - ib * ks, a.up_kper);
  return true;
}

// Down-projection item of tile td and output blocks 2 ob and 2 ob + 1.
template <int ROWS, bool BF>
__device__ __forceinline__ void down_item_of(const FfnArgs& a, int4 td, int ob, Item<ROWS>& it) {
  constexpr int EB = BF ? 2 : 1;
  const int nob = a.d / BLK, nkb = a.I * EB / BLK;
  const int e = td.x, row0 = td.y, nrows = td.z;
  const bool sh = e >= a.E;
  const ExpertPtrs& P = sh ? a.shared : a.routed;
  const size_t eo = sh ? 0 : (size_t)e;
  it.src = make_tile_src<ROWS>(
      [&](int row) {  // a ragged last pair of blocks reads a valid row
        const int o = min(ob * 256 + row, a.d - 1);
        return P.w2 + (eo * a.d + o) * (size_t)a.I * EB;
      },
      [&](int row) { return a.hq + (size_t)(row0 + min(row, nrows - 1)) * a.I * EB; },
      [&](int row) -> const float* {
        return BF ? nullptr : a.hs + (size_t)(row0 + min(row, nrows - 1)) * nkb;
      });
  it.sa0 = BF ? nullptr : P.s2 + (eo * nob + min(2 * ob, nob - 1)) * nkb;
  it.sa1 = BF ? nullptr : P.s2 + (eo * nob + min(2 * ob + 1, nob - 1)) * nkb;
  it.blk = ob;
  it.expert = e;
  it.row0 = row0;
  it.nrows = nrows;
  it.once = (td.w & 1) != 0;
  it.nkb = nkb;
  it.kslice = 0;
}

// Item `item` of the down-projection (tile item / nob2, output blocks
// 2 (item % nob2) and 2 (item % nob2) + 1; with split K, tile
// item / items_per_tile, then output pair and K slice); false past the last
// tile and for padding items.
template <int ROWS, bool BF, bool SPLIT>
__device__ __forceinline__ bool down_item(const FfnArgs& a, int item, Item<ROWS>& it) {
  const int nob2 = (a.d / BLK + 1) >> 1;
  const int ks = SPLIT && a.dn_ks > 1 ? a.dn_ks : 1;
  const int per_tile = items_per_tile(nob2, ks);
  const int tile = item / per_tile;
  const int rem = item - tile * per_tile;
  if (tile >= *a.n_tiles || rem >= nob2 * ks) return false;
  // without split K, tile k of an expert starts its output pairs k (nob2 % 8)
  // further on: items go round-robin over the 8 XCDs, so the item of tile
  // k + 1 that reads a pair's w2 rows then runs on the XCD, and at about the
  // time, of the item of tile k that read them, and that XCD's L2 holds them
  const int4 td = a.tiles[tile];
  const int ob = ks > 1 ? rem / ks : (rem + (td.w >> 1) * (nob2 & 7)) % nob2;
  down_item_of<ROWS, BF>(a, td, ob, it);
  if (ks > 1) item_kslice<ROWS, BF>(it, rem - ob * ks, a.dn_kper);
  return true;
}

// 16-row sub-tiles of this wave that hold rows of the item (wave-uniform)
template <int ROWS>
__device__ __forceinline__ int item_mvalid(const Item<ROWS>& it) {
  const int wr = (threadIdx.x >> 6) >> 2;
  return __builtin_amdgcn_readfirstlane(min(Tile<ROWS>::MVMAX, max(0, (it.nrows - wr * 64 + 15) >> 4)));
}

// Rounding g and u as their exact values round.  A Linear output is an fp32
// sum of d / 128 scaled block products.  Its error is a few units of 2^-24
// times the size of the partial sums (measured against the exact sums on the
// CPU: median 0.5, 99.99th percentile 7, largest 12 units of 2^-24 x the
// largest |sum| of the row among a wave's 32 columns), so when the exact
// value lies near a bf16 rounding midpoint the fp32 sum may round to the
// other neighbour.  A sum v is "uncertain" when it lies within TIE_ULPS x |v|
// x 2^-23 (at least TIE_ULPS of its ulps) plus TIE_ABS x 2^-24 x that row
// maximum of a midpoint; the bf16 values that an interval of that width
// around it rounds to are its candidates.  An uncertain element is
// recomputed exactly only if the outcome depends on its candidates: if they
// give different e4m3 codes of h at the block's scale, or could change the
// block's amax.
constexpr float TIE_ULPS = 4.f;
constexpr float TIE_ABS = 6.f;
// Uncertain elements listed per work item: 1.6 (decode), 54 (prefill) and 76
// (skewed batch) on average.  An element beyond the list keeps its nominal
// rounding.
constexpr int UNC_CAP = 448;

// bf16 h = bf16(silu(g) * u) for bf16 values g and u, evaluated in fp64
// (the exact product rounded once).  Not inlined: it runs rarely, and its
// registers stay out of the epilogue's common path.
__device__ __noinline__ float silu_mul_exact(float g, float u) {
  const double gd = (double)g;
  return bf16_to_f32(f64_to_bf16(gd / (1.0 + exp(-gd)) * (double)u));
}

// The same in fp32, with the fp64 evaluation where the fp32 product lies
// within 8 ulps of a bf16 rounding midpoint, or |g| > 64 (where exp(-g)
// leaves the fp32 range).  exp(-g) = 2^t with t = -g log2(e) split into its
// fp32 rounding th and the remainder tl (an fma gives the product's rounding
// error exactly; the constant's own error is added): 2^th is the hardware
// exp2 (1 ulp) and 2^tl = 1 + tl ln 2 to far below an ulp.  With the
// hardware reciprocal (1 ulp) and four roundings, the fp32 product is within
// 5 ulps of silu(g) u.
__device__ __forceinline__ float silu_mul(float g, float u) {
  constexpr float L2E = 1.44269502f, L2E_LO = 1.92596299e-8f, LN2 = 0.693147182f;
  const float th = -g * L2E;
  const float tl = fmaf(-g, L2E, -th) - g * L2E_LO;
  const float e2 = __builtin_amdgcn_exp2f(th);
  const float e = fmaf(e2, tl * LN2, e2);
  const float h = g * __builtin_amdgcn_rcpf(1.f + e) * u;
  const uint32_t lo = __float_as_uint(h) & 0xFFFFu;
  if (fabsf((float)lo - 32768.f) <= 8.f || fabsf(g) > 64.f) return silu_mul_exact(g, u);
  return round_bf16(h);
}

// Maximum of a non-negative float over lanes l, l ^ 16, l ^ 32 and l ^ 48
// (one row of an MFMA accumulator tile): two gfx950 lane-swap instructions
// instead of LDS permutes.  With both operands equal, permlane16_swap leaves
// rows (0, 0, 2, 2) and (1, 1, 3, 3) of the value in its two results and
// permlane32_swap the halves (lo, lo) and (hi, hi), so each pairwise maximum
// is the maximum with the partner lane.  Non-negative floats order as their
// bits.
typedef unsigned int v2u32 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float rowmax_nonneg(float v) {
  uint32_t b = __float_as_uint(v);
  v2u32 t = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  b = max(t[0], t[1]);
  t = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return __uint_as_float(max(t[0], t[1]));
}

// An uncertain element of the up-projection's epilogue (LDS list entry).
struct UncEntry {
  int key;              // tile row << 8 | h column
  int flags;            // UNC_G, UNC_U: g / u uncertain; UNC_NEED: decided exactly
  float ga, ua;         // the fp32 sums
  float wg, wu;         // half-widths of their candidate intervals
  float hnom;           // h from the nominal roundings
  float hmin, hmax;     // h over the candidates (signed)
  float gx, ux;         // exact bf16 g and u (recomputed components)
  float hfin;           // exact h
};
enum : int { UNC_G = 1, UNC_U = 2, UNC_NEED = 4 };

// The exact (float64) value of one e4m3 Linear output before its bf16
// rounding: the dot product of an e4m3 activation row (one scale per 128
// elements) with an e4m3 weight row (one block scale per 128 inputs).  All
// 64 lanes of the wave call it.  The 16-element partial sums are exact in
// float64 (a product of two e4m3 values has at most 8 significant bits and
// the partial sums span fewer than 53), and each is scaled once by the exact
// product of its two scales.  A lane's loads of up to CH 16-byte chunks of
// each row are issued together (one round trip for rows of up to CH * 1024).
template <int CH>
__device__ __forceinline__ double exact_row_dot(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                                                int d) {
  const int lane = threadIdx.x & 63;
  const int nch = d >> 4;
  double s = 0.0;
  for (int c0 = lane; c0 < nch; c0 += 64 * CH) {
    uint4 xv[CH], wv[CH];
    float xsv[CH], wsv[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = min(c0 + 64 * i, nch - 1);  // past the row's end: its last chunk, not used
      xv[i] = *(const uint4*)(xq + (size_t)c * 16);
      wv[i] = *(const uint4*)(wq + (size_t)c * 16);
      xsv[i] = xs[c >> 3];
      wsv[i] = ws[c >> 3];
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      if (c0 + 64 * i < nch) {
        const uint32_t xw[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w}, ww[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
        double p = 0.0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const v2bf x0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(xw[k], 1.0f, false);
          const v2bf x1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(xw[k], 1.0f, true);
          const v2bf w0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ww[k], 1.0f, false);
          const v2bf w1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ww[k], 1.0f, true);
          p = fma((double)(float)x0[0], (double)(float)w0[0], p);
          p = fma((double)(float)x0[1], (double)(float)w0[1], p);
          p = fma((double)(float)x1[0], (double)(float)w1[0], p);
          p = fma((double)(float)x1[1], (double)(float)w1[1], p);
        }
        s = fma(p, (double)xsv[i] * (double)wsv[i], s);
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  return s;
}

// e4m3 code of h / sc (as the quantiser computes it)
__device__ __forceinline__ uint32_t e4m3_code(float h, float sc) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(h / sc, 0.f, 0, false) & 0xFFu;
}

// Exact g, u and h of the listed elements whose indices `need` holds, one
// wave per element.  row_tok: the token of each tile row (LDS); xq, xs: the
// activation codes and scales (rows by token); w1, w3, s1, s3: the item's
// gate and up weight rows (its first h column) and their K block scales.
// CH: 16-byte chunks per lane in flight (fewer where registers are scarce).
template <int CH>
__device__ __forceinline__ void recompute_listed(UncEntry* ul, const int* need, int n_need, const int* row_tok,
                                                 const uint8_t* xq, const float* xs, const uint8_t* w1,
                                                 const uint8_t* w3, const float* s1, const float* s3, int d) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int nkb = d / BLK;
  for (int k = wave; k < n_need; k += 8) {
    const int i = __builtin_amdgcn_readfirstlane(need[k]);
    const int flags = __builtin_amdgcn_readfirstlane(ul[i].flags);
    const int key = __builtin_amdgcn_readfirstlane(ul[i].key);
    const int tok = __builtin_amdgcn_readfirstlane(row_tok[key >> 8]);
    const uint8_t* xrow = xq + (size_t)tok * d;
    const float* xsrow = xs + (size_t)tok * nkb;
    const size_t wofs = (size_t)(key & 255) * d;
    float gx = ul[i].gx, ux = ul[i].ux;
    if (flags & UNC_G) gx = bf16_to_f32(f64_to_bf16(exact_row_dot<CH>(xrow, xsrow, w1 + wofs, s1, d)));
    if (flags & UNC_U) ux = bf16_to_f32(f64_to_bf16(exact_row_dot<CH>(xrow, xsrow, w3 + wofs, s3, d)));
    if (lane == 0) {
      ul[i].gx = gx;
      ul[i].ux = ux;
      ul[i].hfin = silu_mul_exact(gx, ux);
    }
  }
}

// Up-projection epilogue: h = bf16(silu(bf16 g) * bf16 u) for the wave's 32
// columns of h block it.blk x its 64 rows; e4m3: g, u and h rounded as the
// exact values round (TIE_ULPS), per-row amax over the block's 128 columns
// (4 waves) through `red` (2 KiB of LDS) and a list of uncertain elements
// (up to 22 KiB), then e4m3 h and its scale; bf16: h itself.
template <int ROWS, bool BF, bool COH, bool SPLIT>
__device__ __forceinline__ void up_epilogue(const FfnArgs& a, const Item<ROWS>& it,
                                            const v4f (&acc)[2][2][Tile<ROWS>::MVMAX], float* red) {
  constexpr int MVX = Tile<ROWS>::MVMAX;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  const int wr = wave >> 2, wc = wave & 3;
  const int nib = a.I / BLK;
  if constexpr (SPLIT && !BF) {
    {  // fp32 partials of g and u for K slice (plane) it.kslice: the split
       // instances run only when a.up_ks > 1 or a.up_stream > 0
      const size_t R = (size_t)a.T * a.K + a.T;
#pragma unroll
      for (int m = 0; m < MVX; ++m) {
        const int rr = wr * 64 + 16 * m + r;
        if (rr < it.nrows) {
          float* prow = a.part + ((size_t)it.kslice * R + it.row0 + rr) * 2 * a.I;
#pragma unroll
          for (int gi = 0; gi < 2; ++gi)
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) {
              const v4f v = acc[gi][jt][m];
              *(float4*)(prow + gi * a.I + it.blk * BLK + wc * 32 + jt * 16 + 4 * g) =
                  make_float4(v[0], v[1], v[2], v[3]);
            }
        }
      }
      return;
    }
  }
  if constexpr (BF) {
#pragma unroll
    for (int m = 0; m < MVX; ++m) {
      const int rr = wr * 64 + 16 * m + r;
      if (rr < it.nrows) {
        const size_t row = (size_t)(it.row0 + rr);
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
          uint16_t hb[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float gv = round_bf16(acc[0][jt][m][j]);
            const float uv = round_bf16(acc[1][jt][m][j]);
            hb[j] = f32_to_bf16(gv / (1.f + expf(-gv)) * uv);
          }
          uint2 o;
          o.x = (uint32_t)hb[0] | ((uint32_t)hb[1] << 16);
          o.y = (uint32_t)hb[2] | ((uint32_t)hb[3] << 16);
          st8<COH>((uint16_t*)a.hq + row * a.I + it.blk * BLK + wc * 32 + jt * 16 + 4 * g, o);
        }
      }
    }
    return;
  }
  // g and u as their exact values round (see TIE_ULPS).  LDS after the
  // stage buffers are retired: the per-wave row amax of the certain elements
  // (red), three bounds per tile row (row_hi, row_lo, row_fin: uint bits of
  // non-negative floats, so integer atomicMax orders them), each tile row's
  // token, the list counts and the uncertain elements (UncEntry).  The list
  // is worked by one thread per entry, the exact recomputations by whole
  // waves.
  uint32_t* row_hi = (uint32_t*)(red + 512);
  uint32_t* row_lo = row_hi + 128;
  uint32_t* row_fin = row_lo + 128;
  int* row_tok = (int*)(row_fin + 128);
  int* n_unc_p = row_tok + 128;
  int* n_need_p = n_unc_p + 1;
  int* need = n_unc_p + 4;  // indices of the entries decided exactly
  UncEntry* ul = (UncEntry*)(need + UNC_CAP);
  static_assert(4 * (512 + 4 * 128 + 4 + UNC_CAP) + UNC_CAP * sizeof(UncEntry) <= Tile<ROWS>::template SMEM<false>,
                "the epilogue's LDS must fit in the stage buffers");
  if (threadIdx.x < 384) row_hi[threadIdx.x] = 0u;  // row_hi, row_lo, row_fin
  if (threadIdx.x == 0) n_unc_p[0] = n_unc_p[1] = 0;
  // the lane that copies tile row 64 w + l's activation scales holds its row
  // pointer (xs + token * (d / 128), plus the K offset of a split item)
  if (wave < Tile<ROWS>::SWAVES && wave * 64 + lane < ROWS) row_tok[wave * 64 + lane] = (int)((it.src.s - a.xs) / (a.d / BLK));
  lds_barrier();
  float hv[2][MVX][4] = {};
  uint32_t unc = 0;  // bit (jt MVX + m) 4 + j: the element is listed
#pragma unroll
  for (int m = 0; m < MVX; ++m) {
    if (wr * 64 + 16 * m >= it.nrows) continue;  // a sub-tile without rows (wave-uniform)
    float rmg = 0.f, rmu = 0.f;
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        rmg = fmaxf(rmg, fabsf(acc[0][jt][m][j]));
        rmu = fmaxf(rmu, fabsf(acc[1][jt][m][j]));
      }
    rmg = rowmax_nonneg(rmg);
    rmu = rowmax_nonneg(rmu);
    const float eg = TIE_ABS * 0x1p-24f * rmg, eu = TIE_ABS * 0x1p-24f * rmu;
    const int rr = wr * 64 + 16 * m + r;
    float cmax = 0.f;  // amax of the certain elements
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float ga = acc[0][jt][m][j], ua = acc[1][jt][m][j];
        const float g0 = round_bf16(ga), u0 = round_bf16(ua);
        const float h = silu_mul(g0, u0);
        hv[jt][m][j] = h;
        // distance to the nearer bf16 rounding midpoint (the one between the
        // two bf16 values around the sum; the subtraction is exact) against
        // the half-width of the interval that holds the exact sum (|v| 2^-23
        // is at least one ulp of v)
        const float dg = fabsf(ga - __uint_as_float((__float_as_uint(ga) & 0xFFFF0000u) | 0x8000u));
        const float du = fabsf(ua - __uint_as_float((__float_as_uint(ua) & 0xFFFF0000u) | 0x8000u));
        const bool cg = rr < it.nrows && dg <= fmaf(fabsf(ga), TIE_ULPS * 0x1p-23f, eg);
        const bool cu = rr < it.nrows && du <= fmaf(fabsf(ua), TIE_ULPS * 0x1p-23f, eu);
        if (cg || cu) {
          const int slot = atomicAdd(n_unc_p, 1);
          if (slot < UNC_CAP) {
            unc |= 1u << ((jt * MVX + m) * 4 + j);
            UncEntry& e = ul[slot];
            e.key = (rr << 8) | (wc * 32 + jt * 16 + 4 * g + j);
            e.flags = (cg ? UNC_G : 0) | (cu ? UNC_U : 0);
            e.ga = ga;
            e.ua = ua;
            // plus a margin for the fp32 arithmetic of the interval ends
            e.wg = fmaf(fabsf(ga), (TIE_ULPS + 2.f) * 0x1p-23f, eg);
            e.wu = fmaf(fabsf(ua), (TIE_ULPS + 2.f) * 0x1p-23f, eu);
            continue;
          }
        }
        if (rr < it.nrows) cmax = fmaxf(cmax, fabsf(h));
      }
    cmax = rowmax_nonneg(cmax);
    if (g == 0) red[(wr * 4 + wc) * 64 + 16 * m + r] = cmax;
  }
  lds_barrier();
  const int n_unc = min(__builtin_amdgcn_readfirstlane(*n_unc_p), UNC_CAP);
  int n_need = 0;
  if (n_unc > 0) {  // uniform over the workgroup
    // h over each element's candidates, and the bounds of its row's amax
    for (int i = threadIdx.x; i < n_unc; i += blockDim.x) {
      UncEntry& e = ul[i];
      const float g0 = round_bf16(e.ga), u0 = round_bf16(e.ua);
      const float glo = (e.flags & UNC_G) ? round_bf16(e.ga - e.wg) : g0;
      const float ghi = (e.flags & UNC_G) ? round_bf16(e.ga + e.wg) : g0;
      const float ulo = (e.flags & UNC_U) ? round_bf16(e.ua - e.wu) : u0;
      const float uhi = (e.flags & UNC_U) ? round_bf16(e.ua + e.wu) : u0;
      const float c0 = silu_mul(glo, ulo), c1 = silu_mul(glo, uhi), c2 = silu_mul(ghi, ulo), c3 = silu_mul(ghi, uhi);
      const float hmin = fminf(fminf(c0, c1), fminf(c2, c3)), hmax = fmaxf(fmaxf(c0, c1), fmaxf(c2, c3));
      e.hnom = e.hfin = silu_mul(g0, u0);  // as the owning lane holds it
      e.gx = g0;
      e.ux = u0;
      // h is linear in u and monotone in g away from silu's minimum (g near
      // -1.28): corners bound it; an interval of g that holds more than two
      // bf16 values around that minimum is decided exactly
      const bool wide_min = (e.flags & UNC_G) && glo < -1.2f && ghi > -1.36f &&
                            (__float_as_uint(ghi) - __float_as_uint(glo)) > 0x10000u;
      e.hmin = hmin;
      e.hmax = hmax;
      if (wide_min) e.flags |= UNC_NEED;
      const float lo = (hmin <= 0.f && hmax >= 0.f) ? 0.f : fminf(fabsf(hmin), fabsf(hmax));
      const float hi = wide_min ? INFINITY : fmaxf(fabsf(hmin), fabsf(hmax));
      const int row = e.key >> 8;
      atomicMax(&row_hi[row], __float_as_uint(hi));
      atomicMax(&row_lo[row], __float_as_uint(lo));
    }
    lds_barrier();
    // an element is decided exactly when its row's amax is not settled or its
    // candidates give different e4m3 codes at the row's scale
    for (int i = threadIdx.x; i < n_unc; i += blockDim.x) {
      UncEntry& e = ul[i];
      const int row = e.key >> 8, wrr = row >> 6;
      float cert = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) cert = fmaxf(cert, red[(wrr * 4 + c) * 64 + (row & 63)]);
      const float alo = fmaxf(cert, __uint_as_float(row_lo[row])), ahi = fmaxf(cert, __uint_as_float(row_hi[row]));
      const float sc = alo == 0.f ? 1.f : alo / E4M3_MAX;
      if (ahi > alo || e4m3_code(e.hmin, sc) != e4m3_code(e.hmax, sc)) e.flags |= UNC_NEED;
      if (e.flags & UNC_NEED) need[atomicAdd(n_need_p, 1)] = i;
    }
    lds_barrier();
    n_need = __builtin_amdgcn_readfirstlane(*n_need_p);
    if (n_need > 0) {  // rare: the exact values, kept out of line
      const bool sh = it.expert >= a.E;
      const ExpertPtrs& P = sh ? a.shared : a.routed;
      const size_t wofs = ((sh ? 0 : (size_t)it.expert) * a.I + (size_t)it.blk * BLK) * a.d;
      recompute_listed<ROWS == 32 ? 4 : 8>(ul, need, n_need, row_tok, a.xq, a.xs, P.w1 + wofs, P.w3 + wofs, it.sa0, it.sa1, a.d);
      lds_barrier();
      // the rows' amax over the final values of their uncertain elements
      for (int i = threadIdx.x; i < n_unc; i += blockDim.x)
        atomicMax(&row_fin[ul[i].key >> 8], __float_as_uint(fabsf(ul[i].hfin)));
      lds_barrier();
      if (unc) {  // this lane's listed elements take their final values
        for (int k = 0; k < n_need; ++k) {
          const int i = need[k];
          const int key = ul[i].key;
          const float hf = ul[i].hfin;
#pragma unroll
          for (int m = 0; m < MVX; ++m)
#pragma unroll
            for (int jt = 0; jt < 2; ++jt)
#pragma unroll
              for (int j = 0; j < 4; ++j)
                if (key == (((wr * 64 + 16 * m + r) << 8) | (wc * 32 + jt * 16 + 4 * g + j))) hv[jt][m][j] = hf;
        }
      }
    }
  }
  // A row's amax: its certain elements' and, with no exact recomputation in
  // the tile, its settled lower bound (the bounds of every uncertain element's
  // row then coincide, and hold its nominal h); else the final values'.
  const uint32_t* row_unc = n_need > 0 ? row_fin : row_lo;
#pragma unroll
  for (int m = 0; m < MVX; ++m) {
    const int rr = wr * 64 + 16 * m + r;
    if (rr < it.nrows) {
      float amax = n_unc > 0 ? __uint_as_float(row_unc[rr]) : 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) amax = fmaxf(amax, red[(wr * 4 + c) * 64 + 16 * m + r]);
      const float sc = amax == 0.f ? 1.f : amax / E4M3_MAX;
      const size_t row = (size_t)(it.row0 + rr);
#pragma unroll
      for (int jt = 0; jt < 2; ++jt)
        st<COH>((uint32_t*)(a.hq + row * a.I + it.blk * BLK + wc * 32 + jt * 16 + 4 * g),
                pack4_e4m3(hv[jt][m][0] / sc, hv[jt][m][1] / sc, hv[jt][m][2] / sc, hv[jt][m][3] / sc));
      if (wc == 0 && g == 0) st<COH>(a.hs + row * nib + it.blk, sc);
    }
  }
}

// Down-projection epilogue: the wave's rows of output blocks 2 it.blk and
// 2 it.blk + 1 (the second may lie past d), bf16.
template <int ROWS, bool COH, bool SPLIT>
__device__ __forceinline__ void down_epilogue(const FfnArgs& a, const Item<ROWS>& it,
                                              const v4f (&acc)[2][2][Tile<ROWS>::MVMAX]) {
  constexpr int MVX = Tile<ROWS>::MVMAX;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  const int wr = wave >> 2, wc = wave & 3;
  const int nob = a.d / BLK;
#pragma unroll
  for (int m = 0; m < MVX; ++m) {
    const int rr = wr * 64 + 16 * m + r;
    if (rr < it.nrows) {
      const size_t row = (size_t)(it.row0 + rr);
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        if (2 * it.blk + gi < nob) {
#pragma unroll
          for (int jt = 0; jt < 2; ++jt) {
            const v4f v = acc[gi][jt][m];
            const size_t col = (size_t)(2 * it.blk + gi) * BLK + wc * 32 + jt * 16 + 4 * g;
            if (SPLIT && a.dn_ks > 1) {  // fp32 partial of K slice it.kslice
              const size_t R = (size_t)a.T * a.K + a.T;
              *(float4*)(a.part + ((size_t)it.kslice * R + row) * a.d + col) = make_float4(v[0], v[1], v[2], v[3]);
              continue;
            }
            uint2 o;
            o.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
            o.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
            st8<COH>(a.out + row * a.d + col, o);
          }
        }
      }
    }
  }
}

template <int ROWS>
__device__ __forceinline__ void zero_acc(v4f (&acc)[2][2][Tile<ROWS>::MVMAX]) {
#pragma unroll
  for (int gi = 0; gi < 2; ++gi)
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int m = 0; m < Tile<ROWS>::MVMAX; ++m) acc[gi][jt][m] = v4f{0.f, 0.f, 0.f, 0.f};
}

// All K blocks and the epilogue of one item; smem: Tile<ROWS>::SMEM<BF> bytes of
// LDS.  Called by every thread of a 512-thread workgroup.  COH (for the
// single-launch layer kernel, where other workgroups of the same launch
// produce the activations and consume the outputs): the outputs are written
// with agent-coherent stores and the activation scales copied with
// agent-coherent loads (common.h, ld / st).  Activation rows keep the plain
// policy: every 128-byte line of them comes from one producer, complete
// before any workgroup reads it; a line of scales spans two rows, which may
// belong to tiles finished at different times.  SPLIT: the item may be a K
// slice, whose epilogue stores fp32 partials (FfnArgs: up_ks, dn_ks).
template <bool UP, int ROWS, bool BF, bool COH = false, bool SPLIT = false>
__device__ __forceinline__ void ffn_run_item(const FfnArgs& a, const Item<ROWS>& it, uint8_t* smem) {
  const int nkb = it.nkb;
  v4f acc[2][2][Tile<ROWS>::MVMAX];
  zero_acc<ROWS>(acc);
  run_mainloop<ROWS, BF, COH ? CPOL_SC1 : 0>(smem, it.src, it.sa0, it.sa1, nkb, it.nrows, item_mvalid(it), it.once,
                                             acc);
  if constexpr (UP)
    up_epilogue<ROWS, BF, COH, SPLIT>(a, it, acc, (float*)smem);  // the stage buffers are no longer read
  else
    down_epilogue<ROWS, COH, SPLIT>(a, it, acc);
}

}  // namespace

}  // namespace moe
