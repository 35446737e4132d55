// Device helpers shared by the gfx950 kernels of the MoE layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int BLK = 128;          // FP8 block size of weights and activations
constexpr float E4M3_MAX = 448.f;  // largest finite e4m3fn value

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Round to nearest even bfloat16 (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ float round_bf16(float f) { return bf16_to_f32(f32_to_bf16(f)); }

// bf16 nearest (ties to even) of a double, rounded once: the conversion to
// float rounds to odd (inexact results get their last bit set), which keeps
// the following round-to-nearest-even to bf16 correct.
__device__ __forceinline__ uint16_t f64_to_bf16(double v) {
  float f = (float)v;
  const double back = (double)f;
  if (back != v) {
    uint32_t u = __float_as_uint(f);
    // towards v in magnitude (from a zero f, whose magnitude is below v's,
    // to the smallest subnormal of v's sign)
    if ((u & 1u) == 0u) u += fabs(back) < fabs(v) ? 1u : 0xFFFFFFFFu;
    f = __uint_as_float(u);
  }
  return f32_to_bf16(f);
}

// Whether rounding the fp32 value f to bf16 could go the other way for a
// value within `ulps` fp32 units in the last place of f: the 16 bits that
// the rounding drops lie within `ulps` of the halfway pattern 0x8000.
__device__ __forceinline__ bool near_bf16_tie(float f, uint32_t ulps) {
  return ((__float_as_uint(f) & 0xFFFFu) - (0x8000u - ulps)) < 2u * ulps + 1u;
}

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// A 128-deep e4m3 block operand, decoded to bfloat16 (exact: every e4m3 value
// is a bf16 value) as four 8-element MFMA operands.
struct Frag {
  v8bf k[4];
};

// 32 e4m3 bytes (the lane's share of one 128-deep block) -> Frag.
__device__ __forceinline__ Frag decode_e4m3(v8i q) {
  Frag f;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)q[2 * s], 1.0f, false);
    const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)q[2 * s], 1.0f, true);
    const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)q[2 * s + 1], 1.0f, false);
    const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)q[2 * s + 1], 1.0f, true);
    f.k[s] = v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  }
  return f;
}

// D(16x16) = A(16x128) . B(16x128)^T for one e4m3 block, as four chained
// bf16 MFMAs (products exact, fp32 accumulation).  Lane l ends with
// D[4*(l/16)+j][l%16], j = 0..3.  A and B use the same lane->k mapping.
//
// (The fp8 MFMA forms sum a block with roughly 16 significant bits; the bf16
// path on decoded operands is exact to fp32 rounding, which the layer's
// rounding points -- bf16 g, u, h and an e4m3 re-quantisation of h -- need.)
__device__ __forceinline__ v4f block_dot(const Frag& a, const Frag& b) {
  v4f p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.k[s], b.k[s], p, 0, 0, 0);
  return p;
}

// D += A(16x32 bf16) . B(16x32 bf16)^T
__device__ __forceinline__ v4f mfma_bf16(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Four floats -> four e4m3fn bytes, round to nearest even.  |v| must not
// exceed 464 (the hardware conversion gives NaN above that).
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
  return (uint32_t)v;
}

// 32 bytes of bf16 (16 values: the lane's share of one 64-deep K block) as
// the operands of two 16x16x32 bf16 MFMAs.
struct FragH {
  v8bf k[2];
};

__device__ __forceinline__ FragH as_bf16(v8i q) {
  FragH f;
  f.k[0] = __builtin_bit_cast(v8bf, v4i{q[0], q[1], q[2], q[3]});
  f.k[1] = __builtin_bit_cast(v8bf, v4i{q[4], q[5], q[6], q[7]});
  return f;
}

// Accesses of data that another workgroup of the same launch produces or
// consumes (the single-launch layer kernel).  COH = true: agent-coherent
// loads and stores (relaxed agent-scope atomics: global_load / global_store
// with sc1), which read and write at the point where all XCDs see the same
// memory, so no L2 writeback or invalidation is needed around the completion
// counts that order them.  COH = false: plain accesses.
template <bool COH, typename T>
__device__ __forceinline__ T ld(const T* p) {
  if constexpr (COH)
    return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    return *p;
}

template <bool COH, typename T>
__device__ __forceinline__ void st(T* p, T v) {
  if constexpr (COH)
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}

// 8 and 16 bytes (16-byte aligned for st16); COH: as 8-byte halves.
template <bool COH>
__device__ __forceinline__ void st8(void* p, uint2 v) {
  if constexpr (COH)
    st<true>((uint64_t*)p, __builtin_bit_cast(uint64_t, v));
  else
    *(uint2*)p = v;
}

template <bool COH>
__device__ __forceinline__ void st16(void* p, uint4 v) {
  if constexpr (COH) {
    st<true>((uint64_t*)p, (uint64_t)v.x | ((uint64_t)v.y << 32));
    st<true>((uint64_t*)p + 1, (uint64_t)v.z | ((uint64_t)v.w << 32));
  } else {
    *(uint4*)p = v;
  }
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

}  // namespace moe
