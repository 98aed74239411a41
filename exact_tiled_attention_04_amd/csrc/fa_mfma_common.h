// Device helpers shared by the forward and backward matrix-core kernels
// (gfx950, v_mfma_f32_32x32x16_{bf16,f16}).
#pragma once

#include <hip/hip_runtime.h>

namespace fa {
namespace mfma {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaveSize = 64;

// One 32x32x16 product with fp32 accumulation, and the packing of two fp32
// values into the element type (round to nearest even), per element type.
struct Bf16 {
  static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // two floats -> two bf16 (round to nearest even) in one dword, low first
  static __device__ __forceinline__ unsigned pack2(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(unsigned, v);
  }
};

struct F16 {
  static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ unsigned pack2(float lo, float hi) {
    f16x2 v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(unsigned, v);
  }
};

// Exchange with the lane 32 away: returns the pair in a fixed order (lower
// half-wave's value first) so both lanes compute bit-identical results.
__device__ __forceinline__ void half_pair(float x, float& lo, float& hi) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ s16x4 lds_read_tr(const unsigned short* base, int off) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + off));
}

constexpr int kBufferFlags = 0x00020000;  // raw buffer, 32-bit data format

// Query registers under the sign of the scale (q_sign of the kernel
// parameters): +1 unchanged, -1 every element negated (sign bits flipped),
// 0 zeros.  For eight 16-bit elements and for sixteen E4M3 bytes per u32x4.
__device__ __forceinline__ u32x4 q_signed16(u32x4 x, int sign) {
  const unsigned keep = sign != 0 ? 0xffffffffu : 0u;
  const unsigned flip = sign < 0 ? 0x80008000u : 0u;
  return u32x4{(x[0] & keep) ^ flip, (x[1] & keep) ^ flip, (x[2] & keep) ^ flip, (x[3] & keep) ^ flip};
}
__device__ __forceinline__ u32x4 q_signed8(u32x4 x, int sign) {
  const unsigned keep = sign != 0 ? 0xffffffffu : 0u;
  const unsigned flip = sign < 0 ? 0x80808080u : 0u;
  return u32x4{(x[0] & keep) ^ flip, (x[1] & keep) ^ flip, (x[2] & keep) ^ flip, (x[3] & keep) ^ flip};
}

}  // namespace mfma
}  // namespace fa
