// C ABI of the MoE layer (declared in include/moe.h): argument checks on the
// host, workspace carving, and the launches of the gfx950 kernels.  Nothing
// here allocates device memory or synchronises the host.
#include <math.h>

#include <algorithm>
#include <mutex>

#include "../../include/moe.h"
#include "common.h"
#include "kernels.h"

using namespace moe;

namespace {

#define MOE_TRY(expr)            \
  do {                           \
    const int st_ = (expr);      \
    if (st_ != MOE_OK) return st_; \
  } while (0)

constexpr size_t WS_ALIGN = 256;
constexpr int MAX_FEATURES = 32768;  // keeps every row offset and grid size well inside int32

struct Layout {
  size_t zpart, idx, w, chunk_cnt, chunk_off, counts, offsets, row_token, pair_row, tiles, n_tiles, xq, xs, hq,
      hs, rows, total;
};

size_t align_up(size_t v) { return (v + WS_ALIGN - 1) & ~(WS_ALIGN - 1); }

Layout layout(const moe_dims& dm, int64_t T) {
  Layout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  const size_t E = dm.n_experts, K = dm.topk, d = dm.d_model, I = dm.inter, t = (size_t)T;
  const size_t rows = t * K + t;
  const size_t nchunks = (t + PERM_CHUNK - 1) / PERM_CHUNK;
  // the tile list is sized for the narrower of the e4m3 and bf16 tiles (more tiles)
  const int NT = std::min(ffn_tile_rows(T), ffn_tile_rows(T, false, true));
  L.zpart = take((size_t)gate_ksplit(T, dm.d_model, dm.n_experts) * t * E * 4);
  L.idx = take(t * K * 4);
  L.w = take(t * K * 4);
  L.chunk_cnt = take(nchunks * E * 4);
  L.chunk_off = take(nchunks * E * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.row_token = take(rows * 4);
  L.pair_row = take(t * K * 4);
  L.tiles = take((size_t)ffn_max_tiles(T, dm.topk, dm.n_experts, NT) * sizeof(int4));
  L.n_tiles = take(4);
  L.xq = take(t * d);
  L.xs = take(t * (d / BLK) * 4);
  L.hq = take(rows * I * 2);  // e4m3 h, or bf16 h with bf16 expert weights
  L.hs = take(rows * (I / BLK) * 4);
  L.rows = take(rows * d * 2);
  L.total = off;
  return L;
}

// Single-launch forward: the control block first, then what the steps pass on.
struct FusedLayout {
  size_t ctl, zpart, idx, w, counts, offsets, row_token, pair_row, tiles, n_tiles, xq, xs, hq, hs, rows, total;
};

FusedLayout fused_layout(const moe_dims& dm, int64_t T) {
  FusedLayout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  const size_t E = dm.n_experts, K = dm.topk, d = dm.d_model, I = dm.inter, t = (size_t)T;
  const size_t rows = t * K + t;
  const DecodeShape sh = decode_shape((int)T, dm.d_model, dm.inter, dm.n_experts, dm.topk);
  L.ctl = take(DEC_CTL_INTS * 4);
  L.zpart = take((size_t)2 * sh.gate_kz * t * E * 4);
  L.idx = take(t * K * 4);
  L.w = take(t * K * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.row_token = take(rows * 4);
  L.pair_row = take(t * K * 4);
  L.tiles = take((size_t)sh.max_tiles * sizeof(int4));
  L.n_tiles = take(4);
  L.xq = take(t * d);
  L.xs = take(t * (d / BLK) * 4);
  L.hq = take(rows * I);
  L.hs = take(rows * (I / BLK) * 4);
  L.rows = take(rows * d * 2);
  L.total = off;
  return L;
}

// Dense MLP: xq, xs, the tile list and h.
struct MlpLayout {
  size_t xq, xs, tiles, n_tiles, hq, hs, part, total;
  int up_ks, up_kper, dn_ks, dn_kper;  // split K (part: the larger set of fp32 partial planes)
  int up_stream, up_planes;            // stream-K up-projection (ffn_dense_ksplit)
};

MlpLayout mlp_layout(int d, int I, int64_t T) {
  MlpLayout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  const size_t t = (size_t)T;
  L.xq = take(t * d);
  L.xs = take(t * (d / BLK) * 4);
  L.tiles = take((size_t)ffn_max_tiles(T, 0, 0, ffn_tile_rows(T, true)) * sizeof(int4));
  L.n_tiles = take(4);
  L.hq = take(t * I);
  L.hs = take(t * (I / BLK) * 4);
  ffn_dense_ksplit(T, d, I, &L.up_ks, &L.up_kper, &L.dn_ks, &L.dn_kper, &L.up_stream, &L.up_planes);
  const size_t up_part = (size_t)L.up_planes * t * 2 * I * 4;
  const size_t dn_part = L.dn_ks > 1 ? (size_t)L.dn_ks * t * d * 4 : 0;
  L.part = take(std::max(up_part, dn_part));
  L.total = off;
  return L;
}

int check_mlp(int32_t d, int32_t I, int64_t T) {
  if (d <= 0 || I <= 0 || T < 0) return MOE_ERR_INVALID_ARG;
  if (d % BLK != 0 || I % BLK != 0 || d > MAX_FEATURES || I > MAX_FEATURES) return MOE_ERR_UNSUPPORTED;
  if (T > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int check_dims(const moe_dims* p) {
  if (!p) return MOE_ERR_INVALID_ARG;
  const moe_dims& d = *p;
  if (d.d_model <= 0 || d.inter <= 0 || d.n_experts <= 0 || d.n_groups <= 0 || d.topk_groups <= 0 || d.topk <= 0)
    return MOE_ERR_INVALID_ARG;
  if (d.n_experts % d.n_groups != 0 || d.topk_groups > d.n_groups) return MOE_ERR_INVALID_ARG;
  if (d.topk > d.topk_groups * (d.n_experts / d.n_groups)) return MOE_ERR_INVALID_ARG;
  if (!isfinite(d.route_scale)) return MOE_ERR_INVALID_ARG;
  if (d.d_model % BLK != 0 || d.inter % BLK != 0) return MOE_ERR_UNSUPPORTED;
  if (d.d_model > MAX_FEATURES || d.inter > MAX_FEATURES) return MOE_ERR_UNSUPPORTED;
  if (d.n_experts > 256 || d.n_experts % 16 != 0) return MOE_ERR_UNSUPPORTED;
  if (d.n_groups > 64 || d.n_experts / d.n_groups < 2) return MOE_ERR_UNSUPPORTED;
  if (d.topk > 32) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int check_tokens(const moe_dims& d, int64_t T) {
  if (T < 0) return MOE_ERR_INVALID_ARG;
  // permuted rows (T*K routed + T shared) are indexed with int32
  if (T > (int64_t)(0x7fffffff / (d.topk + 1))) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int check_fused(const moe_dims* dims, int64_t T) {
  MOE_TRY(check_dims(dims));
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (T > DEC_MAX_TOKENS) return MOE_ERR_UNSUPPORTED;
  if (T > 0) {
    const DecodeShape sh = decode_shape((int)T, dims->d_model, dims->inter, dims->n_experts, dims->topk);
    if (DEC_CTL_UP + sh.max_tiles > DEC_CTL_INTS) return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int check_experts(const moe_experts* x) {
  if (!x || !x->w1 || !x->w3 || !x->w2 || !x->s1 || !x->s3 || !x->s2) return MOE_ERR_INVALID_ARG;
  if (!aligned(x->w1, 16) || !aligned(x->w3, 16) || !aligned(x->w2, 16)) return MOE_ERR_ALIGN;
  if (!aligned(x->s1, 4) || !aligned(x->s3, 4) || !aligned(x->s2, 4)) return MOE_ERR_ALIGN;
  return MOE_OK;
}

ExpertPtrs ptrs(const moe_experts& x) { return ExpertPtrs{x.w1, x.w3, x.w2, x.s1, x.s3, x.s2}; }

int check_experts_bf16(const moe_experts_bf16* x) {
  if (!x || !x->w1 || !x->w3 || !x->w2) return MOE_ERR_INVALID_ARG;
  if (!aligned(x->w1, 16) || !aligned(x->w3, 16) || !aligned(x->w2, 16)) return MOE_ERR_ALIGN;
  return MOE_OK;
}

ExpertPtrs ptrs(const moe_experts_bf16& x) {
  return ExpertPtrs{(const uint8_t*)x.w1, (const uint8_t*)x.w3, (const uint8_t*)x.w2, nullptr, nullptr, nullptr};
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

}  // namespace

extern "C" {

size_t moe_workspace_size(const moe_dims* dims, int64_t tokens) {
  if (check_dims(dims) != MOE_OK || check_tokens(*dims, tokens) != MOE_OK) return 0;
  return layout(*dims, tokens).total;
}

int moe_gate(const moe_dims* dims, int64_t tokens, const uint16_t* x, const float* gate_w, const float* gate_b,
             int32_t* idx, float* w, void* workspace, size_t workspace_bytes, void* stream) {
  MOE_TRY(check_dims(dims));
  MOE_TRY(check_tokens(*dims, tokens));
  if (tokens == 0) return MOE_OK;
  if (!x || !gate_w || !gate_b || !idx || !w) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(gate_w, 16) || !aligned(gate_b, 4) || !aligned(idx, 4) || !aligned(w, 4))
    return MOE_ERR_ALIGN;
  const Layout L = layout(*dims, tokens);
  if (!workspace || workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (!aligned(workspace, WS_ALIGN)) return MOE_ERR_ALIGN;
  const moe_dims& d = *dims;
  return hip_status(launch_gate(x, gate_w, gate_b, (int)tokens, d.d_model, d.n_experts, d.n_groups, d.topk_groups,
                                d.topk, d.route_scale, at<float>(workspace, L.zpart),
                                gate_ksplit(tokens, d.d_model, d.n_experts), idx, w, (hipStream_t)stream));
}

int moe_permute(const moe_dims* dims, int64_t tokens, const int32_t* idx, const uint16_t* x, int32_t* counts,
                int32_t* offsets, int32_t* row_token, int32_t* pair_row, uint8_t* xq, float* xs, void* workspace,
                size_t workspace_bytes, void* stream) {
  MOE_TRY(check_dims(dims));
  MOE_TRY(check_tokens(*dims, tokens));
  if (tokens == 0) return MOE_OK;
  if (!idx || !x || !counts || !offsets || !row_token || !pair_row || (!xq) != (!xs)) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(idx, 4) || !aligned(counts, 4) || !aligned(offsets, 4) ||
      !aligned(row_token, 4) || !aligned(pair_row, 4) || !aligned(xs, 4))
    return MOE_ERR_ALIGN;
  const Layout L = layout(*dims, tokens);
  if (!workspace || workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (!aligned(workspace, WS_ALIGN)) return MOE_ERR_ALIGN;
  const moe_dims& d = *dims;
  return hip_status(launch_permute(idx, x, (int)tokens, d.d_model, d.n_experts, d.topk,
                                   at<int32_t>(workspace, L.chunk_cnt), at<int32_t>(workspace, L.chunk_off), counts,
                                   offsets, row_token, pair_row, xq, xs, (hipStream_t)stream));
}

int moe_grouped_ffn(const moe_dims* dims, int64_t tokens, const moe_experts* routed, const moe_experts* shared,
                    const int32_t* offsets, const int32_t* row_token, const uint8_t* xq, const float* xs,
                    uint16_t* out, void* workspace, size_t workspace_bytes, void* stream) {
  MOE_TRY(check_dims(dims));
  MOE_TRY(check_tokens(*dims, tokens));
  if (tokens == 0) return MOE_OK;
  MOE_TRY(check_experts(routed));
  if (shared) MOE_TRY(check_experts(shared));
  if (!offsets || !row_token || !xq || !xs || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned(xq, 16) || !aligned(out, 16) || !aligned(offsets, 4) || !aligned(row_token, 4) || !aligned(xs, 4))
    return MOE_ERR_ALIGN;
  const Layout L = layout(*dims, tokens);
  if (!workspace || workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (!aligned(workspace, WS_ALIGN)) return MOE_ERR_ALIGN;
  const moe_dims& d = *dims;
  const ExpertPtrs rp = ptrs(*routed);
  ExpertPtrs sp;
  if (shared) sp = ptrs(*shared);
  return hip_status(launch_ffn(rp, shared ? &sp : nullptr, (int)tokens, d.d_model, d.inter, d.n_experts, d.topk,
                               offsets, row_token, xq, xs, at<int4>(workspace, L.tiles),
                               at<int32_t>(workspace, L.n_tiles), at<uint8_t>(workspace, L.hq),
                               at<float>(workspace, L.hs), out, (hipStream_t)stream));
}

int moe_grouped_ffn_bf16(const moe_dims* dims, int64_t tokens, const moe_experts_bf16* routed,
                         const moe_experts_bf16* shared, const int32_t* offsets, const int32_t* row_token,
                         const uint16_t* x, uint16_t* out, void* workspace, size_t workspace_bytes, void* stream) {
  MOE_TRY(check_dims(dims));
  MOE_TRY(check_tokens(*dims, tokens));
  if (tokens == 0) return MOE_OK;
  MOE_TRY(check_experts_bf16(routed));
  if (shared) MOE_TRY(check_experts_bf16(shared));
  if (!offsets || !row_token || !x || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(offsets, 4) || !aligned(row_token, 4)) return MOE_ERR_ALIGN;
  const Layout L = layout(*dims, tokens);
  if (!workspace || workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (!aligned(workspace, WS_ALIGN)) return MOE_ERR_ALIGN;
  const moe_dims& d = *dims;
  const ExpertPtrs rp = ptrs(*routed);
  ExpertPtrs sp;
  if (shared) sp = ptrs(*shared);
  return hip_status(launch_ffn(rp, shared ? &sp : nullptr, (int)tokens, d.d_model, d.inter, d.n_experts, d.topk,
                               offsets, row_token, (const uint8_t*)x, nullptr, at<int4>(workspace, L.tiles),
                               at<int32_t>(workspace, L.n_tiles), at<uint8_t>(workspace, L.hq), nullptr, out,
                               (hipStream_t)stream, nullptr, true));
}

int moe_combine(const moe_dims* dims, int64_t tokens, const int32_t* idx, const float* w, const int32_t* pair_row,
                const uint16_t* rows, int32_t has_shared, uint16_t* delta, void* stream) {
  MOE_TRY(check_dims(dims));
  MOE_TRY(check_tokens(*dims, tokens));
  if (tokens == 0) return MOE_OK;
  if (!idx || !w || !pair_row || !rows || !delta) return MOE_ERR_INVALID_ARG;
  if (!aligned(rows, 16) || !aligned(delta, 16) || !aligned(idx, 4) || !aligned(w, 4) || !aligned(pair_row, 4))
    return MOE_ERR_ALIGN;
  const moe_dims& d = *dims;
  return hip_status(launch_combine(idx, w, pair_row, rows, has_shared ? 1 : 0, (int)tokens, d.topk, d.n_experts,
                                   d.d_model, delta, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// The fused forward.  ev: NULL or MOE_FORWARD_EVENTS events, recorded before
// the gate, before the permutation, before the up-projection, before the
// down-projection, before the combine and after it.  routed / shared: the
// expert weights, e4m3 with scales or (bf16 = true) bf16 without.
int forward_impl(const moe_dims* dims, const float* gate_w, const float* gate_b, const ExpertPtrs& routed,
                 const ExpertPtrs& shared, bool bf16, int64_t tokens, const uint16_t* x, uint16_t* delta,
                 int32_t* idx_out, float* w_out, void* workspace, size_t workspace_bytes, hipStream_t s,
                 hipEvent_t* ev) {
  if (!gate_w || !gate_b || !x || !delta) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(delta, 16) || !aligned(gate_w, 16) || !aligned(gate_b, 4) ||
      (idx_out && !aligned(idx_out, 4)) || (w_out && !aligned(w_out, 4)))
    return MOE_ERR_ALIGN;
  const Layout L = layout(*dims, tokens);
  if (!workspace || workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (!aligned(workspace, WS_ALIGN)) return MOE_ERR_ALIGN;
  const moe_dims& d = *dims;
  const int T = (int)tokens;
  int32_t* idx = idx_out ? idx_out : at<int32_t>(workspace, L.idx);
  float* w = w_out ? w_out : at<float>(workspace, L.w);
  int32_t* offsets = at<int32_t>(workspace, L.offsets);
  int32_t* row_token = at<int32_t>(workspace, L.row_token);
  int32_t* pair_row = at<int32_t>(workspace, L.pair_row);
  // e4m3 weights take the quantised x; bf16 weights take x itself
  uint8_t* xq = bf16 ? nullptr : at<uint8_t>(workspace, L.xq);
  float* xs = bf16 ? nullptr : at<float>(workspace, L.xs);
  uint16_t* rows = at<uint16_t>(workspace, L.rows);
  record_event(ev, 0, s);
  MOE_TRY(hip_status(launch_gate(x, gate_w, gate_b, T, d.d_model, d.n_experts, d.n_groups, d.topk_groups, d.topk,
                                 d.route_scale, at<float>(workspace, L.zpart),
                                 gate_ksplit(tokens, d.d_model, d.n_experts), idx, w, s)));
  record_event(ev, 1, s);
  // small batches: the permutation kernel also writes the FFN tile list
  const PlanArgs plan{at<int4>(workspace, L.tiles), at<int32_t>(workspace, L.n_tiles),
                      ffn_tile_rows(tokens, false, bf16), 1, ffn_plan_cap(tokens, d.topk, d.n_experts, true, bf16)};
  bool planned = false;
  MOE_TRY(hip_status(launch_permute(idx, x, T, d.d_model, d.n_experts, d.topk, at<int32_t>(workspace, L.chunk_cnt),
                                    at<int32_t>(workspace, L.chunk_off), at<int32_t>(workspace, L.counts), offsets,
                                    row_token, pair_row, xq, xs, s, &plan, &planned)));
  MOE_TRY(hip_status(launch_ffn(routed, &shared, T, d.d_model, d.inter, d.n_experts, d.topk, offsets, row_token,
                                bf16 ? (const uint8_t*)x : xq, xs, at<int4>(workspace, L.tiles),
                                at<int32_t>(workspace, L.n_tiles), at<uint8_t>(workspace, L.hq),
                                bf16 ? nullptr : at<float>(workspace, L.hs), rows, s, ev ? ev + 2 : nullptr, bf16, 0,
                                -1, planned)));
  const int st = hip_status(launch_combine(idx, w, pair_row, rows, 1, T, d.topk, d.n_experts, d.d_model, delta, s));
  record_event(ev, 5, s);
  return st;
}

int forward_bf16(const moe_dims* dims, const moe_weights_bf16* weights, int64_t tokens, const uint16_t* x,
                 uint16_t* delta, int32_t* idx_out, float* w_out, void* workspace, size_t workspace_bytes,
                 hipStream_t s, hipEvent_t* ev) {
  MOE_TRY(check_dims(dims));
  MOE_TRY(check_tokens(*dims, tokens));
  if (tokens == 0) return MOE_OK;
  if (!weights) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_experts_bf16(&weights->routed));
  MOE_TRY(check_experts_bf16(&weights->shared));
  return forward_impl(dims, weights->gate_w, weights->gate_b, ptrs(weights->routed), ptrs(weights->shared), true,
                      tokens, x, delta, idx_out, w_out, workspace, workspace_bytes, s, ev);
}

int take_events(void* const* stage_events, hipEvent_t* ev) {
  if (!stage_events) return MOE_ERR_INVALID_ARG;
  for (int i = 0; i < MOE_FORWARD_EVENTS; ++i) ev[i] = (hipEvent_t)stage_events[i];  // NULL: not recorded
  return MOE_OK;
}

int forward_fp8(const moe_dims* dims, const moe_weights* weights, int64_t tokens, const uint16_t* x,
                uint16_t* delta, int32_t* idx_out, float* w_out, void* workspace, size_t workspace_bytes,
                hipStream_t s, hipEvent_t* ev) {
  MOE_TRY(check_dims(dims));
  MOE_TRY(check_tokens(*dims, tokens));
  if (tokens == 0) return MOE_OK;
  if (!weights) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_experts(&weights->routed));
  MOE_TRY(check_experts(&weights->shared));
  return forward_impl(dims, weights->gate_w, weights->gate_b, ptrs(weights->routed), ptrs(weights->shared), false,
                      tokens, x, delta, idx_out, w_out, workspace, workspace_bytes, s, ev);
}

}  // namespace

extern "C" {

int moe_forward(const moe_dims* dims, const moe_weights* weights, int64_t tokens, const uint16_t* x,
                uint16_t* delta, int32_t* idx_out, float* w_out, void* workspace, size_t workspace_bytes,
                void* stream) {
  return forward_fp8(dims, weights, tokens, x, delta, idx_out, w_out, workspace, workspace_bytes,
                     (hipStream_t)stream, nullptr);
}

int moe_forward_timed(const moe_dims* dims, const moe_weights* weights, int64_t tokens, const uint16_t* x,
                      uint16_t* delta, int32_t* idx_out, float* w_out, void* workspace, size_t workspace_bytes,
                      void* stream, void* const* stage_events) {
  hipEvent_t ev[MOE_FORWARD_EVENTS];
  MOE_TRY(take_events(stage_events, ev));
  return forward_fp8(dims, weights, tokens, x, delta, idx_out, w_out, workspace, workspace_bytes,
                     (hipStream_t)stream, ev);
}

int moe_forward_bf16(const moe_dims* dims, const moe_weights_bf16* weights, int64_t tokens, const uint16_t* x,
                     uint16_t* delta, int32_t* idx_out, float* w_out, void* workspace, size_t workspace_bytes,
                     void* stream) {
  return forward_bf16(dims, weights, tokens, x, delta, idx_out, w_out, workspace, workspace_bytes,
                      (hipStream_t)stream, nullptr);
}

int moe_forward_bf16_timed(const moe_dims* dims, const moe_weights_bf16* weights, int64_t tokens, const uint16_t* x,
                           uint16_t* delta, int32_t* idx_out, float* w_out, void* workspace, size_t workspace_bytes,
                           void* stream, void* const* stage_events) {
  hipEvent_t ev[MOE_FORWARD_EVENTS];
  MOE_TRY(take_events(stage_events, ev));
  return forward_bf16(dims, weights, tokens, x, delta, idx_out, w_out, workspace, workspace_bytes,
                      (hipStream_t)stream, ev);
}

int moe_forward_shard(const moe_dims* dims, const moe_weights* weights, int64_t tokens, int32_t expert_begin,
                      int32_t expert_end, int32_t with_shared, const uint16_t* x, const int32_t* idx, const float* w,
                      float* y_partial, void* workspace, size_t workspace_bytes, void* stream) {
  MOE_TRY(check_dims(dims));
  MOE_TRY(check_tokens(*dims, tokens));
  const moe_dims& d = *dims;
  if (expert_begin < 0 || expert_end > d.n_experts || expert_begin >= expert_end) return MOE_ERR_INVALID_ARG;
  if (tokens == 0) return MOE_OK;
  if (!weights || !x || !idx || !w || !y_partial) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_experts(&weights->routed));
  if (with_shared) MOE_TRY(check_experts(&weights->shared));
  if (!aligned(x, 16) || !aligned(y_partial, 16) || !aligned(idx, 4) || !aligned(w, 4)) return MOE_ERR_ALIGN;
  const Layout L = layout(d, tokens);
  if (!workspace || workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (!aligned(workspace, WS_ALIGN)) return MOE_ERR_ALIGN;
  const hipStream_t s = (hipStream_t)stream;
  const int T = (int)tokens;
  int32_t* offsets = at<int32_t>(workspace, L.offsets);
  int32_t* row_token = at<int32_t>(workspace, L.row_token);
  int32_t* pair_row = at<int32_t>(workspace, L.pair_row);
  uint8_t* xq = at<uint8_t>(workspace, L.xq);
  float* xs = at<float>(workspace, L.xs);
  uint16_t* rows = at<uint16_t>(workspace, L.rows);
  MOE_TRY(hip_status(launch_permute(idx, x, T, d.d_model, d.n_experts, d.topk, at<int32_t>(workspace, L.chunk_cnt),
                                    at<int32_t>(workspace, L.chunk_off), at<int32_t>(workspace, L.counts), offsets,
                                    row_token, pair_row, xq, xs, s)));
  const ExpertPtrs rp = ptrs(weights->routed);
  ExpertPtrs sp;
  if (with_shared) sp = ptrs(weights->shared);
  MOE_TRY(hip_status(launch_ffn(rp, with_shared ? &sp : nullptr, T, d.d_model, d.inter, d.n_experts, d.topk, offsets,
                                row_token, xq, xs, at<int4>(workspace, L.tiles), at<int32_t>(workspace, L.n_tiles),
                                at<uint8_t>(workspace, L.hq), at<float>(workspace, L.hs), rows, s, nullptr, false,
                                expert_begin, expert_end)));
  return hip_status(launch_combine_partial(idx, w, pair_row, rows, with_shared ? 1 : 0, T, d.topk, expert_begin,
                                           expert_end, d.d_model, y_partial, s));
}

}  // extern "C"

namespace {

// The workspace of moe_forward_no_workspace: one array per GPU, for callers
// that cannot allocate.  In host code `scratch` names a host-side stand-in;
// its device address comes from hipGetSymbolAddress, looked up once per
// device with that device current and kept in scratch_dev.
static __device__ __align__(256) uint8_t scratch[MOE_STATIC_WORKSPACE_BYTES];
constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_dev[SCRATCH_MAX_DEVICES] = {};

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= SCRATCH_MAX_DEVICES) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    scratch_dev[dev] = p;
  }
  *out = scratch_dev[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_forward_no_workspace(const moe_dims* dims, const moe_weights* weights, int64_t tokens, const uint16_t* x,
                             uint16_t* delta, int32_t* idx_out, float* w_out, void* stream) {
  MOE_TRY(check_dims(dims));
  MOE_TRY(check_tokens(*dims, tokens));
  if (tokens == 0) return MOE_OK;
  if (layout(*dims, tokens).total > MOE_STATIC_WORKSPACE_BYTES) return MOE_ERR_UNSUPPORTED;
  void* ws = nullptr;
  MOE_TRY(scratch_address(&ws));
  return forward_fp8(dims, weights, tokens, x, delta, idx_out, w_out, ws, MOE_STATIC_WORKSPACE_BYTES,
                     (hipStream_t)stream, nullptr);
}

size_t moe_forward_fused_workspace_size(const moe_dims* dims, int64_t tokens) {
  if (check_fused(dims, tokens) != MOE_OK || tokens == 0) return 0;
  return fused_layout(*dims, tokens).total;
}

int moe_forward_fused(const moe_dims* dims, const moe_weights* weights, int64_t tokens, const uint16_t* x,
                      uint16_t* delta, int32_t* idx_out, float* w_out, void* workspace, size_t workspace_bytes,
                      void* stream) {
  MOE_TRY(check_fused(dims, tokens));
  if (tokens == 0) return MOE_OK;
  if (!weights || !weights->gate_w || !weights->gate_b || !x || !delta) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_experts(&weights->routed));
  MOE_TRY(check_experts(&weights->shared));
  if (!aligned(x, 16) || !aligned(delta, 16) || !aligned(weights->gate_w, 16) || !aligned(weights->gate_b, 4) ||
      (idx_out && !aligned(idx_out, 4)) || (w_out && !aligned(w_out, 4)))
    return MOE_ERR_ALIGN;
  const FusedLayout L = fused_layout(*dims, tokens);
  if (!workspace || workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (!aligned(workspace, WS_ALIGN)) return MOE_ERR_ALIGN;
  const moe_dims& d = *dims;
  const int T = (int)tokens;
  const DecodeShape sh = decode_shape(T, d.d_model, d.inter, d.n_experts, d.topk);
  DecodeBufs b;
  b.ctl = at<int>(workspace, L.ctl);
  b.zpart = at<float>(workspace, L.zpart);
  b.idx = idx_out ? idx_out : at<int32_t>(workspace, L.idx);
  b.w = w_out ? w_out : at<float>(workspace, L.w);
  b.counts = at<int32_t>(workspace, L.counts);
  b.offsets = at<int32_t>(workspace, L.offsets);
  b.row_token = at<int32_t>(workspace, L.row_token);
  b.pair_row = at<int32_t>(workspace, L.pair_row);
  b.tiles = at<int4>(workspace, L.tiles);
  b.n_tiles = at<int32_t>(workspace, L.n_tiles);
  b.xq = at<uint8_t>(workspace, L.xq);
  b.xs = at<float>(workspace, L.xs);
  b.hq = at<uint8_t>(workspace, L.hq);
  b.hs = at<float>(workspace, L.hs);
  b.rows = at<uint16_t>(workspace, L.rows);
  return hip_status(launch_decode(sh, ptrs(weights->routed), ptrs(weights->shared), x, weights->gate_w,
                                  weights->gate_b, T, d.d_model, d.inter, d.n_experts, d.n_groups, d.topk_groups,
                                  d.topk, d.route_scale, b, delta, (hipStream_t)stream));
}

int moe_forward_fused_status(const void* workspace, void* stream) {
  if (!workspace) return MOE_ERR_INVALID_ARG;
  int32_t st = 0;
  const hipStream_t s = (hipStream_t)stream;
  if (hipMemcpyAsync(&st, static_cast<const int32_t*>(workspace) + DEC_CTL_STATUS, sizeof(st),
                     hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return MOE_ERR_HIP;
  return st == 0 ? MOE_OK : MOE_ERR_STALLED;
}

int moe_add_rmsnorm(int32_t d, int64_t tokens, const uint16_t* x, uint16_t* residual, const float* gain, float eps,
                    uint16_t* out, void* stream) {
  if (d <= 0 || tokens < 0 || !(eps >= 0.f) || !isfinite(eps)) return MOE_ERR_INVALID_ARG;
  if (d % BLK != 0 || d > 16384) return MOE_ERR_UNSUPPORTED;
  if (tokens > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
  if (tokens == 0) return MOE_OK;
  if (!x || !residual || !gain || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(residual, 16) || !aligned(gain, 16) || !aligned(out, 16)) return MOE_ERR_ALIGN;
  return hip_status(launch_add_rmsnorm(x, residual, gain, eps, d, tokens, out, (hipStream_t)stream));
}

size_t moe_mlp_workspace_size(int32_t d_model, int32_t inter, int64_t tokens) {
  if (check_mlp(d_model, inter, tokens) != MOE_OK) return 0;
  return mlp_layout(d_model, inter, tokens).total;
}

int moe_mlp(int32_t d_model, int32_t inter, int64_t tokens, const moe_experts* mlp, const uint16_t* x,
            uint16_t* out, void* workspace, size_t workspace_bytes, void* stream) {
  MOE_TRY(check_mlp(d_model, inter, tokens));
  if (tokens == 0) return MOE_OK;
  MOE_TRY(check_experts(mlp));
  if (!x || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(out, 16)) return MOE_ERR_ALIGN;
  const MlpLayout L = mlp_layout(d_model, inter, tokens);
  if (!workspace || workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (!aligned(workspace, WS_ALIGN)) return MOE_ERR_ALIGN;
  const hipStream_t s = (hipStream_t)stream;
  uint8_t* xq = at<uint8_t>(workspace, L.xq);
  float* xs = at<float>(workspace, L.xs);
  // one dense expert: no routed experts, rows are tokens; the quantisation
  // launch also writes its tile list
  const PlanArgs plan{at<int4>(workspace, L.tiles), at<int32_t>(workspace, L.n_tiles),
                      ffn_tile_rows(tokens, true), 1, 0};
  MOE_TRY(hip_status(launch_quant(x, tokens, d_model, xq, xs, s, &plan)));
  const ExpertPtrs p = ptrs(*mlp);
  const FfnSplit split{at<float>(workspace, L.part), L.up_ks, L.up_kper, L.dn_ks, L.dn_kper, L.up_stream};
  return hip_status(launch_ffn(p, &p, (int)tokens, d_model, inter, 0, 0, nullptr, nullptr, xq, xs, plan.tiles,
                               plan.n_tiles, at<uint8_t>(workspace, L.hq), at<float>(workspace, L.hs), out, s, nullptr,
                               false, 0, -1, true, &split));
}

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported dimensions";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_ALIGN: return "misaligned pointer";
    case MOE_ERR_HIP: return "HIP launch failed";
    case MOE_ERR_STALLED: return "a wait in the single-launch forward gave up (outputs not valid)";
    default: return "unknown status";
  }
}

}  // extern "C"
