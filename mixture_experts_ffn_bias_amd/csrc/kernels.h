// Host-side launchers of the gfx950 kernels (one per kernel file).  Each
// returns the hipError_t of its launch(es).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

struct ExpertPtrs {
  const uint8_t* w1;
  const uint8_t* w3;
  const uint8_t* w2;
  const float* s1;
  const float* s3;
  const float* s2;
};

// tokens per permutation chunk (one workgroup of the count / scatter kernels)
constexpr int PERM_CHUNK = 256;

// gate.hip
int gate_ksplit(int64_t T, int d, int E);
hipError_t launch_gate(const uint16_t* x, const float* gate_w, const float* gate_b, int T, int d, int E,
                       int G, int TG, int K, float route_scale, float* zpart, int ksplit, int32_t* idx,
                       float* w, hipStream_t s);

// permute.hip
// The FFN tile list for all E experts, written alongside the permutation
// when the batch fits one permutation chunk (see launch_ffn).
struct PlanArgs {
  int4* tiles;
  int32_t* n_tiles;
  int tile_rows;
  int has_shared;
  int cap;
};
// plan (may be NULL): also write the tile list when T <= PERM_CHUNK; *planned
// (may be NULL) tells whether it was written.
hipError_t launch_permute(const int32_t* idx, const uint16_t* x, int T, int d, int E, int K,
                          int32_t* chunk_cnt, int32_t* chunk_off, int32_t* counts, int32_t* offsets,
                          int32_t* row_token, int32_t* pair_row, uint8_t* xq, float* xs, hipStream_t s,
                          const PlanArgs* plan = nullptr, bool* planned = nullptr);
// per-128-block e4m3 quantisation of T rows of d bf16 values.  dense_plan
// (may be NULL): also write the tile list of one dense expert over the T
// rows (the MLP; tiles, n_tiles and tile_rows are read), as launch_ffn's
// `planned` expects it.
hipError_t launch_quant(const uint16_t* x, int64_t T, int d, uint8_t* xq, float* xs, hipStream_t s,
                        const PlanArgs* dense_plan = nullptr);

// Record ev[i] on s unless the array or that entry is NULL (stage timing).
inline void record_event(hipEvent_t* ev, int i, hipStream_t s) {
  if (ev && ev[i]) (void)hipEventRecord(ev[i], s);
}

// ffn.hip
// rows per FFN tile for this token count (dense: the MLP; bf16: bf16 expert weights)
int ffn_tile_rows(int64_t T, bool dense = false, bool bf16 = false);
int64_t ffn_max_tiles(int64_t T, int K, int E, int tile_rows);
// E = K = 0 with `shared` set and row_token NULL runs one dense expert over
// rows 0..T-1 (offsets is then not read).
// ev: NULL, or three events recorded before the up-projection, before the
// down-projection and after it (the tile plan precedes ev[0]); a NULL entry
// is not recorded.
// bf16: the expert weights are bf16 without scales; xq is then the bf16
// input x, hq receives bf16 h ([rows][I]) and xs, hs and the scale pointers
// are unused.
// [e_lo, e_hi) (e_hi < 0: E): the routed experts to run; `routed` then holds
// exactly those experts (expert e_lo first).  Rows of other experts are left
// untouched.  planned: the tile list is already in tiles / n_tiles (written
// by launch_permute with a PlanArgs), so no plan kernel runs.
// split: NULL, or split K of the projections (ffn_dense_ksplit).
struct FfnSplit {
  float* part;  // max(up planes * 2 I, dn_ks * d) * (T*K + T) fp32 partials
  int up_ks, up_kper, dn_ks, dn_kper;
  int up_stream;  // > 0: stream-K up-projection in runs of up_stream K blocks (one dense expert), up_ks ignored
};
hipError_t launch_ffn(const ExpertPtrs& routed, const ExpertPtrs* shared, int T, int d, int I, int E,
                      int K, const int32_t* offsets, const int32_t* row_token, const uint8_t* xq,
                      const float* xs, int4* tiles, int32_t* n_tiles, uint8_t* hq, float* hs,
                      uint16_t* out, hipStream_t s, hipEvent_t* ev = nullptr, bool bf16 = false,
                      int e_lo = 0, int e_hi = -1, bool planned = false, const FfnSplit* split = nullptr);
// Split K of the dense MLP's projections (one expert over T rows, e4m3) for
// batches with too few items to occupy the chip: slices of *_kper K blocks,
// *_ks = 1 where splitting does not pay.
// *up_stream > 0 instead selects the stream-K up-projection (runs of
// *up_stream K blocks; *up_ks = 1); *up_planes: the partial planes it needs
// (the up-projection's, either way).
void ffn_dense_ksplit(int64_t T, int d, int I, int* up_ks, int* up_kper, int* dn_ks, int* dn_kper, int* up_stream,
                      int* up_planes);
// routed tiles the plan may write (the tile list holds ffn_max_tiles entries)
int ffn_plan_cap(int64_t T, int K, int E, bool has_shared, bool bf16 = false);

// combine.hip
hipError_t launch_combine(const int32_t* idx, const float* w, const int32_t* pair_row, const uint16_t* rows,
                          int has_shared, int T, int K, int E, int d, uint16_t* delta, hipStream_t s);
// The fp32 partial sum of the experts in [e_lo, e_hi) (+ the shared rows when
// has_shared), in ascending expert order, without the final bf16 rounding.
hipError_t launch_combine_partial(const int32_t* idx, const float* w, const int32_t* pair_row,
                                  const uint16_t* rows, int has_shared, int T, int K, int e_lo, int e_hi, int d,
                                  float* y, hipStream_t s);

// decode.hip: the whole layer in one launch for T <= DEC_MAX_TOKENS (e4m3
// expert weights).  The control block (DEC_CTL_INTS ints at the start of the
// workspace) must be zero before the first launch on it; every launch leaves
// it zero except DEC_CTL_STATUS, which then holds 1 if a wait gave up (the
// outputs are not valid) and 0 otherwise.
constexpr int DEC_MAX_TOKENS = 64;
// Control words, each count in a cache line of its own (many workgroups poll
// some of them while others add to them).
enum : int {
  DEC_CTL_QUANT = 0,      // quantisation items done
  DEC_CTL_GATE = 32,      // router partial items done
  DEC_CTL_SELECT = 64,    // selection items done
  DEC_CTL_PLAN = 96,      // permutation + tile list done
  DEC_CTL_DOWN = 128,     // down-projection items done
  DEC_CTL_FINISHED = 160, // workgroups finished
  DEC_CTL_STALLED = 192,  // a wait gave up
  DEC_CTL_STATUS = 224,   // status of the last completed launch
  DEC_CTL_DTICKET = 256,  // down-projection items handed out
  DEC_CTL_UP = 288,       // DEC_CTL_UP + tile: up-projection items of that tile done
};
constexpr int DEC_CTL_INTS = 1024;

struct DecodeShape {
  int max_tiles, nsh, gate_kz, gate_kchunk, comb_parts;
  int b_gate, b_sup, b_sel, b_plan, b_rup, b_down, b_comb, b_end;  // item ranges
};
DecodeShape decode_shape(int T, int d, int I, int E, int K);

struct DecodeBufs {
  int* ctl;
  float* zpart;  // 2 gate_kz planes of [T][E]
  int32_t* idx;
  float* w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* row_token;
  int32_t* pair_row;
  int4* tiles;
  int32_t* n_tiles;
  uint8_t* xq;
  float* xs;
  uint8_t* hq;
  float* hs;
  uint16_t* rows;
};
hipError_t launch_decode(const DecodeShape& sh, const ExpertPtrs& routed, const ExpertPtrs& shared,
                         const uint16_t* x, const float* gate_w, const float* gate_b, int T, int d, int I, int E,
                         int G, int TG, int K, float route_scale, const DecodeBufs& bufs, uint16_t* delta,
                         hipStream_t s);

// norm.hip
hipError_t launch_add_rmsnorm(const uint16_t* x, uint16_t* residual, const float* gain, float eps, int d,
                              int64_t T, uint16_t* out, hipStream_t s);

}  // namespace moe
