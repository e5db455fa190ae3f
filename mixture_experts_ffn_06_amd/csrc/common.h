// Device helpers shared by the libmoe kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr int kQBlock = 128;       // fp8 block edge (weights 128x128, rows x 128)
constexpr float kE4M3Max = 448.0f;

// Storage-format tags used as template parameters (kMXFP4 / kMXFP8: OCP MX
// FP4 E2M1 / FP8 E4M3 weights with an E8M0 scale per 32 elements along K;
// activations bf16).
enum : int { kF32 = 0, kBF16 = 1, kFP8 = 2, kMXFP4 = 3, kMXFP8 = 4 };
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __uint_as_float(static_cast<uint32_t>(u) << 16);
}

// fp32 -> bf16, round to nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u)
    return static_cast<uint16_t>((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// One OCP e4m3fn code -> fp32 (hardware convert).
__device__ __forceinline__ float fp8_to_f32(uint32_t code) {
  return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(code), 0);
}

// Two fp32 -> two e4m3fn codes (round to nearest even) in the low 16 bits.
// Inputs here never exceed 448 in magnitude by more than one fp32 ulp,
// which rounds to 448.
__device__ __forceinline__ int fp8_pack2(float a, float b) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
}

// Eight e4m3fn codes (two 32-bit words, lowest byte first) as their exact
// bf16 values: every e4m3 value, subnormals included, is a bf16 value, and a
// scale operand of 1.0 leaves the conversion unscaled.
__device__ __forceinline__ bf16x8_t e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  const bf16x2_t q0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2_t q1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2_t q2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2_t q3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8_t{q0[0], q0[1], q1[0], q1[1], q2[0], q2[1], q3[0], q3[1]};
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Load one element of a storage format as fp32 (fp8: the raw code value;
// the caller applies block scales).
template <int DT>
__device__ __forceinline__ float load_as_f32(const void *base, size_t i) {
  if constexpr (DT == kF32) {
    return static_cast<const float *>(base)[i];
  } else if constexpr (DT == kBF16) {
    return bf16_to_f32(static_cast<const uint16_t *>(base)[i]);
  } else {
    return fp8_to_f32(static_cast<const uint8_t *>(base)[i]);
  }
}

template <int DT> struct StorageBytes { static constexpr int value = DT == kF32 ? 4 : (DT == kBF16 ? 2 : 1); };

}  // namespace moe
