/*
 * moe.h -- C ABI of the MI355X (gfx950) DeepSeek-V3.2-Exp MoE layer forward.
 *
 * The layer maps x [tokens, d_model] (bf16) to its MoE update of the same
 * shape ("DeepSeek-V3.2-Exp · MoE update": output expression and shape;
 * "DeepSeek-V3.2-Exp · Add shared output": formula).  The steps are exposed
 * one by one (gate, permute, grouped FFN, combine) and fused (moe_forward);
 * a fused residual-add RMSNorm ("MoE update", rmsnorm excerpt) precedes the
 * layer when blocks are stacked.
 *
 * Conventions shared by every entry point:
 *  - All array arguments are DEVICE pointers (HIP device memory) unless the
 *    comment says "host".  Structs passed by pointer are host memory, read
 *    during the call only.
 *  - The caller owns every buffer.  The library allocates nothing, keeps no
 *    state between calls (moe_forward_fused keeps counters in the caller's
 *    workspace) and never synchronises the host (moe_forward_fused_status
 *    does, by design): work is enqueued
 *    on `stream` (a hipStream_t; NULL = the default stream) and a return of
 *    MOE_OK means "enqueued".  Calls on different streams are independent as
 *    long as their buffers (workspace included) do not overlap.
 *  - bf16 tensors are passed as uint16_t (the bit pattern).  FP8 tensors are
 *    OCP e4m3fn codes (uint8_t), with one float32 scale per 128x128 block.
 *  - Row-major layouts throughout.  d_model and inter must be multiples of
 *    128 and at most 32768; n_experts <= 256 and a multiple of 16; experts
 *    per group >= 2; n_groups <= 64; topk <= 32.
 *  - Errors: arguments are checked on the host before anything is enqueued;
 *    a negative moe_status is returned and nothing runs.  A failed launch
 *    returns MOE_ERR_HIP.  tokens == 0 is a valid no-op.
 *  - Routing indices must lie in [0, n_experts) and be distinct within a
 *    token.  Out-of-range indices are clamped into range and duplicates give
 *    unspecified (but finite-memory, non-faulting) results.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null pointer, negative size, inconsistent dims */
  MOE_ERR_UNSUPPORTED = -2, /* dims outside what the kernels implement */
  MOE_ERR_WORKSPACE = -3,   /* workspace missing or smaller than moe_workspace_size() */
  MOE_ERR_ALIGN = -4,       /* a pointer is not aligned as documented */
  MOE_ERR_HIP = -5,         /* a HIP launch failed */
  MOE_ERR_STALLED = -6      /* moe_forward_fused_status: a wait inside the last call gave up */
} moe_status;

/* Layer shape (host struct).  DeepSeek-V3.2-Exp: {7168, 256, 8, 4, 8, 2048, 2.5}. */
typedef struct {
  int32_t d_model;     /* hidden size d ("MoE update": shape [B, T, 7168]) */
  int32_t n_experts;   /* routed experts E ("Gate projection" breadcrumb: 256 routed experts) */
  int32_t n_groups;    /* expert groups G; group g holds experts [g*E/G, (g+1)*E/G) */
  int32_t topk_groups; /* groups kept per token */
  int32_t topk;        /* experts selected per token K */
  int32_t inter;       /* expert hidden size ("Gate projection": 2048 expert d_ff) */
  float route_scale;   /* factor applied to the normalised router weights */
} moe_dims;

/* n SwiGLU experts with FP8 Linear layers ("Gate projection", expert and Linear
 * excerpts): w1, w3 map d -> inter, w2 maps inter -> d; weights are [out, in]. */
typedef struct {
  const uint8_t* w1; /* e4m3fn [n][inter][d]    (16-byte aligned) */
  const uint8_t* w3; /* e4m3fn [n][inter][d]    (16-byte aligned) */
  const uint8_t* w2; /* e4m3fn [n][d][inter]    (16-byte aligned) */
  const float* s1;   /* fp32  [n][inter/128][d/128] */
  const float* s3;   /* fp32  [n][inter/128][d/128] */
  const float* s2;   /* fp32  [n][d/128][inter/128] */
} moe_experts;

/* All parameters of one MoE layer.  The 256x7168 router weight plus a
 * 256-element router bias are what the pages' count of 11,320,164,608 MoE
 * parameters leaves after 257 experts ("MoE transformer block", parameter
 * accounting table). */
typedef struct {
  const float* gate_w; /* fp32 [E][d] router weight */
  const float* gate_b; /* fp32 [E]    router bias, added to the scores for selection only */
  moe_experts routed;  /* n = E */
  moe_experts shared;  /* n = 1, applied to every token ("Add shared output") */
} moe_weights;

/* n SwiGLU experts with bf16 Linear layers.  A Linear whose weight elements
 * are wider than one byte carries no scale ("Gate projection", Linear
 * excerpt: the constructor registers no scale parameter then); such a Linear
 * multiplies the bf16 activation itself, without quantisation.
 * Layout as moe_experts, elements bf16 (uint16_t bit patterns). */
typedef struct {
  const uint16_t* w1; /* bf16 [n][inter][d]    (16-byte aligned) */
  const uint16_t* w3; /* bf16 [n][inter][d]    (16-byte aligned) */
  const uint16_t* w2; /* bf16 [n][d][inter]    (16-byte aligned) */
} moe_experts_bf16;

/* All parameters of one MoE layer with bf16 expert weights. */
typedef struct {
  const float* gate_w;     /* fp32 [E][d] router weight */
  const float* gate_b;     /* fp32 [E]    router bias */
  moe_experts_bf16 routed; /* n = E */
  moe_experts_bf16 shared; /* n = 1 */
} moe_weights_bf16;

/* Workspace bytes that any single entry point below (including moe_forward)
 * needs for `tokens` tokens.  Returns 0 for invalid dims. */
size_t moe_workspace_size(const moe_dims* dims, int64_t tokens);

/* Router: the gate call of the moe-forward excerpt on "MoE update", which
 * returns each token's routing weights and expert indices.
 *   x       bf16 [T][d]   (16-byte aligned)
 *   gate_w  fp32 [E][d]   (16-byte aligned), gate_b fp32 [E]
 *   idx     int32 [T][K]  out: selected experts, descending biased score
 *   w       fp32  [T][K]  out: sigmoid scores of idx normalised to sum 1, times route_scale
 * Scores s = sigmoid(x . gate_w^T) are computed with fp32 accumulation; the
 * selection uses b = s + gate_b: groups ranked by the sum of their two
 * largest b, the top topk_groups groups kept, then the top K of b among the
 * kept experts.  Ties go to the lower index.  Needs the workspace. */
int moe_gate(const moe_dims* dims, int64_t tokens, const uint16_t* x, const float* gate_w,
             const float* gate_b, int32_t* idx, float* w, void* workspace, size_t workspace_bytes,
             void* stream);

/* Token counting and expert-contiguous order (the moe-forward excerpt on
 * "MoE update" counts the tokens of each expert and gathers them expert by
 * expert), plus the FP8 activation quantisation the expert Linear layers
 * consume.
 *   idx        int32 [T][K]      routing from moe_gate
 *   x          bf16  [T][d]      (16-byte aligned)
 *   counts     int32 [E]         out: rows per expert
 *   offsets    int32 [E+1]       out: exclusive prefix sum of counts
 *   row_token  int32 [T*K + T]   out: token of each permuted row; rows of expert e
 *                                are [offsets[e], offsets[e+1]) in ascending token
 *                                order; rows [T*K, T*K+T) are the shared expert's
 *                                and hold 0..T-1
 *   pair_row   int32 [T][K]      out: row of (token t, choice k)
 *   xq         e4m3  [T][d]      out: per-128-block quantised x (16-byte aligned)
 *   xs         fp32  [T][d/128]  out: block scales, amax/448 (1 for an all-zero block)
 * xq and xs may both be NULL: the quantisation is then skipped (bf16-weight
 * experts take x itself).  Needs the workspace. */
int moe_permute(const moe_dims* dims, int64_t tokens, const int32_t* idx, const uint16_t* x,
                int32_t* counts, int32_t* offsets, int32_t* row_token, int32_t* pair_row,
                uint8_t* xq, float* xs, void* workspace, size_t workspace_bytes, void* stream);

/* Grouped expert FFN over the permuted rows ("Gate projection", expert
 * excerpt: SwiGLU of the two input projections taken in fp32, the product
 * cast back to the input dtype, then the output projection):
 * for every row r of expert e (and every shared-expert row),
 *   g = bf16(Q(x) . W1_e^T), u = bf16(Q(x) . W3_e^T), h = bf16(silu(g) * u),
 *   out[r] = bf16(Q(h) . W2_e^T)
 * with Q the per-128-block e4m3 activation quantiser and W the block-scaled
 * FP8 weights.
 *   routed, shared  expert weights (shared may be NULL: shared rows are then skipped)
 *   offsets, row_token, xq, xs   from moe_permute
 *   out             bf16 [T*K + T][d] out: one row per permuted row (16-byte aligned)
 * Needs the workspace. */
int moe_grouped_ffn(const moe_dims* dims, int64_t tokens, const moe_experts* routed,
                    const moe_experts* shared, const int32_t* offsets, const int32_t* row_token,
                    const uint8_t* xq, const float* xs, uint16_t* out, void* workspace,
                    size_t workspace_bytes, void* stream);

/* moe_grouped_ffn for bf16-weight experts: the same SwiGLU with bf16 Linear
 * layers and no quantisation,
 *   g = bf16(x . W1_e^T), u = bf16(x . W3_e^T), h = bf16(silu(g) * u), out[r] = bf16(h . W2_e^T)
 * (fp32 accumulation; bf16 MFMAs on the operands as given).
 *   routed, shared  bf16 expert weights (shared may be NULL: shared rows are then skipped)
 *   offsets, row_token   from moe_permute (which may skip its quantisation)
 *   x               bf16 [T][d] the layer input (16-byte aligned)
 *   out             bf16 [T*K + T][d] out, one row per permuted row (16-byte aligned)
 * Needs the workspace. */
int moe_grouped_ffn_bf16(const moe_dims* dims, int64_t tokens, const moe_experts_bf16* routed,
                         const moe_experts_bf16* shared, const int32_t* offsets, const int32_t* row_token,
                         const uint16_t* x, uint16_t* out, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Router-weighted combine plus shared output ("MoE update", moe-forward
 * excerpt: each expert's rows, scaled by their routing weights, are added to
 * an fp32 accumulator expert by expert in ascending order, then the shared
 * expert's output, then the sum is cast back to x's dtype):
 *   delta[t] = bf16( sum over k in ascending idx[t][k] of w[t][k] * rows[pair_row[t][k]]
 *                    + rows[T*K + t] )     accumulated in fp32.
 *   rows    bf16 [T*K + T][d] from moe_grouped_ffn (16-byte aligned)
 *   delta   bf16 [T][d] out (16-byte aligned)
 * Pass has_shared = 0 to leave the shared rows out. */
int moe_combine(const moe_dims* dims, int64_t tokens, const int32_t* idx, const float* w,
                const int32_t* pair_row, const uint16_t* rows, int32_t has_shared,
                uint16_t* delta, void* stream);

/* The whole layer ("DeepSeek-V3.2-Exp · MoE update": the moe-forward excerpt
 * flattens x to [tokens, d], calls the gate, counts the tokens per expert,
 * runs each selected expert on its tokens and adds the router-weighted
 * outputs into an fp32 accumulator in ascending expert id, adds the shared
 * expert's output for every token, and casts the sum back to x's dtype, the
 * page's output expression and shape; "Add shared output", formula):
 * gate -> permute -> grouped FFN -> combine, enqueued with no host
 * synchronisation (the per-expert counts stay on the device).
 *   x       bf16 [T][d] (16-byte aligned)
 *   delta   bf16 [T][d] out, the layer's update (16-byte aligned; must not alias x)
 *   idx_out int32 [T][K], w_out fp32 [T][K]: out, the routing, when non-NULL
 * Needs moe_workspace_size(dims, T) bytes of workspace (256-byte aligned). */
int moe_forward(const moe_dims* dims, const moe_weights* weights, int64_t tokens,
                const uint16_t* x, uint16_t* delta, int32_t* idx_out, float* w_out,
                void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the device array that moe_forward_no_workspace uses in place of a
 * workspace (one per GPU the library runs on, held until the process ends). */
#define MOE_STATIC_WORKSPACE_BYTES ((size_t)32 << 20)

/* moe_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments and the same result as moe_forward, without a workspace
 * argument.  The workspace is a file-scope device array of
 * MOE_STATIC_WORKSPACE_BYTES on each GPU (its address is looked up once per
 * device, on the first call with that device current); the call allocates
 * nothing.  tokens must satisfy moe_workspace_size(dims, tokens) <=
 * MOE_STATIC_WORKSPACE_BYTES (up to 181 tokens at the DeepSeek-V3.2-Exp
 * shape), else MOE_ERR_UNSUPPORTED is returned before anything runs.  Every
 * call on one GPU uses that GPU's array: calls that overlap in time on one GPU
 * (other streams, other threads) race and give undefined results; order them.
 * No part of the array needs to start zeroed. */
int moe_forward_no_workspace(const moe_dims* dims, const moe_weights* weights, int64_t tokens,
                             const uint16_t* x, uint16_t* delta, int32_t* idx_out, float* w_out,
                             void* stream);

/* Number of events moe_forward_timed records. */
#define MOE_FORWARD_EVENTS 6

/* moe_forward that also records stage_events[0..5] (hipEvent_t handles the
 * caller created, host array) on `stream`: before the gate, before the
 * permutation, before the up-projection (w1/w3, SwiGLU, h quantisation),
 * before the down-projection (w2), before the combine, and after it.  A NULL
 * entry is not recorded (each recorded event adds a little time to the
 * step, so a caller times only the stages it needs); a NULL array is
 * MOE_ERR_INVALID_ARG.  For per-kernel timing; the computation is identical
 * to moe_forward. */
int moe_forward_timed(const moe_dims* dims, const moe_weights* weights, int64_t tokens,
                      const uint16_t* x, uint16_t* delta, int32_t* idx_out, float* w_out,
                      void* workspace, size_t workspace_bytes, void* stream,
                      void* const* stage_events);

/* moe_forward with bf16 expert weights (moe_grouped_ffn_bf16 in place of the
 * quantised FFN; the router is the same). */
int moe_forward_bf16(const moe_dims* dims, const moe_weights_bf16* weights, int64_t tokens,
                     const uint16_t* x, uint16_t* delta, int32_t* idx_out, float* w_out,
                     void* workspace, size_t workspace_bytes, void* stream);

/* moe_forward_bf16 recording the stage events of moe_forward_timed. */
int moe_forward_bf16_timed(const moe_dims* dims, const moe_weights_bf16* weights, int64_t tokens,
                           const uint16_t* x, uint16_t* delta, int32_t* idx_out, float* w_out,
                           void* workspace, size_t workspace_bytes, void* stream,
                           void* const* stage_events);

/* One rank's share of an expert-parallel layer ("MoE update", moe-forward
 * excerpt: a rank runs only its contiguous slice of the experts, and the
 * ranks' y are summed by an all-reduce before the cast to the input dtype).
 *   expert_begin, expert_end  the rank's routed experts, 0 <= begin < end <= E
 *   weights->routed           holds exactly those end - begin experts, expert_begin first
 *   with_shared               1: add the shared expert (one rank of the group does);
 *                             0: weights->shared is not read
 *   x      bf16 [T][d]  all tokens (16-byte aligned)
 *   idx, w int32 / fp32 [T][K]  the routing of every token (moe_gate)
 *   y_partial  fp32 [T][d] out: sum over k with idx[t][k] in [begin, end), in ascending
 *              expert id, of w[t][k] * expert(x[t]) (+ the shared expert), fp32, unrounded
 *              (16-byte aligned)
 * Summing y_partial over ranks that cover [0, E) once (the shared expert on one of
 * them) and rounding to bf16 gives moe_forward's output up to the fp32 order of the
 * cross-rank sum.  Needs moe_workspace_size(dims, T). */
int moe_forward_shard(const moe_dims* dims, const moe_weights* weights, int64_t tokens,
                      int32_t expert_begin, int32_t expert_end, int32_t with_shared,
                      const uint16_t* x, const int32_t* idx, const float* w, float* y_partial,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes moe_forward_fused needs; 0 when the call is not supported
 * for these dims and tokens (tokens must lie in [1, 64]). */
size_t moe_forward_fused_workspace_size(const moe_dims* dims, int64_t tokens);

/* moe_forward in ONE kernel launch, for small batches (1 <= tokens <= 64,
 * e4m3 expert weights): router, permutation, the up- and down-projections of
 * the routed and shared experts and the combine ("MoE update", moe-forward
 * excerpt, every step) run as one grid whose workgroups wait on each other's
 * completion counts in device memory.  Same arguments and the same result as
 * moe_forward (the router adds its K-split partial logits in a different
 * grouping, so a logit may differ in its last fp32 bits).
 * Workspace: moe_forward_fused_workspace_size(dims, tokens) bytes, 256-byte
 * aligned.  Its first 4096 bytes carry completion counts from call to call:
 * they must be zero before the first call on a workspace (zero the whole
 * workspace once), and every completed call leaves them zero except the
 * status word that moe_forward_fused_status reads.  Calls sharing a
 * workspace must be ordered (one stream).  A wait that cannot complete gives
 * up after a bounded time instead of hanging; the call's outputs are then not
 * valid and moe_forward_fused_status reports MOE_ERR_STALLED. */
int moe_forward_fused(const moe_dims* dims, const moe_weights* weights, int64_t tokens,
                      const uint16_t* x, uint16_t* delta, int32_t* idx_out, float* w_out,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Status of the last moe_forward_fused call on `workspace` enqueued on
 * `stream`: waits for the stream (the one call here that synchronises the
 * host), then returns MOE_OK or MOE_ERR_STALLED (MOE_ERR_HIP if the wait or
 * the copy fails). */
int moe_forward_fused_status(const void* workspace, void* stream);

/* Fused residual add + RMSNorm ("MoE update", rmsnorm excerpt, residual branch):
 *   r = float(x) + float(residual);  residual <- bf16(r);
 *   out = bf16(gain * r * rsqrt(mean(r^2) + eps))
 * The normalisation is evaluated in fp64 and rounded once to bf16, so the
 * result does not depend on the reduction order.
 *   x, residual, out  bf16 [T][d] (16-byte aligned; out may alias x); gain fp32 [d].
 * d must be a multiple of 128 and at most 16384.  No workspace. */
int moe_add_rmsnorm(int32_t d, int64_t tokens, const uint16_t* x, uint16_t* residual,
                    const float* gain, float eps, uint16_t* out, void* stream);

/* Workspace bytes moe_mlp needs for `tokens` tokens.  Returns 0 for invalid sizes. */
size_t moe_mlp_workspace_size(int32_t d_model, int32_t inter, int64_t tokens);

/* Dense MLP of the blocks that precede the MoE blocks ("DeepSeek-V3.2-Exp ·
 * MoE update", block excerpt: the first few blocks build a dense MLP of the
 * model width where the others build the MoE).  The pages print neither the
 * MLP's body nor its hidden width; it is taken to be the SwiGLU of one
 * expert in the same FP8 form ("Gate projection", expert and Linear excerpts):
 *   out[t] = bf16(Q(h) . W2^T),  h = bf16(silu(bf16(Q(x[t]) . W1^T)) * bf16(Q(x[t]) . W3^T))
 * with Q the per-128-block e4m3 activation quantiser of moe_grouped_ffn.
 *   mlp   one expert's weights (n = 1): w1, w3 [inter][d_model], w2 [d_model][inter]
 *   x     bf16 [T][d_model] (16-byte aligned)
 *   out   bf16 [T][d_model] out (16-byte aligned; must not alias x)
 * d_model and inter: multiples of 128, at most 32768.  Needs
 * moe_mlp_workspace_size(d_model, inter, T) bytes of workspace (256-byte aligned).
 * The workspace holds Q(x), the tile list, Q(h) and, for batches too small
 * to occupy the GPU, fp32 partial sums of the two products over slices of
 * their K range.  The partials are added in a fixed order, so repeated calls
 * give identical results.  Its contents are scratch between calls. */
int moe_mlp(int32_t d_model, int32_t inter, int64_t tokens, const moe_experts* mlp, const uint16_t* x,
            uint16_t* out, void* workspace, size_t workspace_bytes, void* stream);

/* Static description of a status code. */
const char* moe_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
