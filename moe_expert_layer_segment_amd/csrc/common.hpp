// Shared device helpers of the gfx950 MoE-LoRA kernels: element types, MFMA
// fragment operations and small integer utilities.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace moelora {

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int int4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// Element traits.  A "frag" is the 8 consecutive K elements one lane feeds to a
// 16x16 MFMA block per 32-deep K step: one v_mfma_f32_16x16x32_bf16 for bf16,
// eight v_mfma_f32_16x16x4_f32 for fp32 (the K order inside a 32-step is
// permuted identically for both operands, which leaves the dot product intact).
template <typename T> struct Elt;

template <> struct Elt<bf16_t> {
  typedef bf16x8 frag;
  static constexpr int kChunk = 8;  // elements per 16-byte chunk
  __device__ static inline floatx4 mma(const frag& a, const frag& b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static inline bf16_t from_float(float v) { return (bf16_t)v; }
  __device__ static inline float to_float(bf16_t v) { return (float)v; }
  __device__ static inline frag zero() {
    frag z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = (bf16_t)0.0f;
    return z;
  }
};

template <> struct Elt<float> {
  typedef floatx8 frag;
  static constexpr int kChunk = 4;
  __device__ static inline floatx4 mma(const frag& a, const frag& b, floatx4 c) {
#pragma unroll
    for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], c, 0, 0, 0);
    return c;
  }
  __device__ static inline float from_float(float v) { return v; }
  __device__ static inline float to_float(float v) { return v; }
  __device__ static inline frag zero() {
    frag z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = 0.0f;
    return z;
  }
};

// Load one frag (8 consecutive elements, 16 B for bf16 / 32 B for fp32) from
// global memory.
template <typename T>
__device__ inline typename Elt<T>::frag load_frag_global(const T* p) {
  return *reinterpret_cast<const typename Elt<T>::frag*>(p);
}

// SiLU(v) = v * sigmoid(v) = v / (1 + e^-v), with e^-v evaluated as
// 2^(-v * log2(e)) on the hardware exp2 unit and the division as a multiply
// by the hardware reciprocal (about 1 ulp; for e^-v = inf it gives 0).
// The weighted down rows (z) of a bf16 layer, stored for the combine: each
// fp32 value rounded to its top 24 bits (sign, exponent and 15 explicit
// significand bits, round to nearest even: a relative error of at most 2^-16),
// four values packed into three 32-bit words.  Infinities and NaNs are cut,
// not rounded, so they stay what they are.
__device__ inline uint32_t fp24_bits(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const uint32_t r = (u & 0x7F800000u) == 0x7F800000u ? u : u + 0x7Fu + ((u >> 8) & 1u);
  return r >> 8;
}
__device__ inline u32x3 fp24_pack4(floatx4 v) {
  const uint32_t a = fp24_bits(v[0]), b = fp24_bits(v[1]), c = fp24_bits(v[2]), d = fp24_bits(v[3]);
  u32x3 w;
  w[0] = a | (b << 24);
  w[1] = (b >> 8) | (c << 16);
  w[2] = (c >> 16) | (d << 8);
  return w;
}
__device__ inline floatx4 fp24_unpack4(u32x3 w) {
  floatx4 v;
  v[0] = __builtin_bit_cast(float, w[0] << 8);
  v[1] = __builtin_bit_cast(float, (w[1] << 16) | ((w[0] >> 16) & 0xFF00u));
  v[2] = __builtin_bit_cast(float, (w[2] << 24) | ((w[1] >> 8) & 0xFFFF00u));
  v[3] = __builtin_bit_cast(float, w[2] & 0xFFFFFF00u);
  return v;
}

__device__ inline float silu_f(float v) {
  const float kLog2e = 1.4426950408889634f;
  float e = __builtin_amdgcn_exp2f(-v * kLog2e);
  return v * __builtin_amdgcn_rcpf(1.0f + e);
}

__device__ inline int lane_id() { return threadIdx.x & 63; }

// Device-side precondition checks of MOE_LORA_DEBUG builds: a violated
// precondition sets its bit in one device word (a vector atomic OR; the word's
// address is passed to the kernels, null in release builds, where the checks
// are compiled out).  The bits are those of MOE_LORA_DEBUG_* in moe_lora.h.
__device__ inline void debug_flag(uint32_t* word, uint32_t bit) {
#ifdef MOE_LORA_DEBUG
  if (word) atomicOr(word, bit);
#else
  (void)word;
  (void)bit;
#endif
}

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0..N-1.  Used
// where an index selects accumulator registers, so the body is always
// instantiated per index (never left as a runtime loop over a register array).
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

}  // namespace moelora
