// Matrix-core (MFMA) operand helpers shared by the query kernels
// (pa_prefill.hip) and the grouped-query decode kernel (pa_decode_mfma.hip),
// gfx950: the 16x16x32 / 16x16x16 fp16 and bf16 products, the operand words
// of the P.V product and the deferred-rescaling bound.
#pragma once

#include "pa_device.h"

namespace pa {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));
typedef short s4_t __attribute__((ext_vector_type(4)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <typename T>
struct Mfma;

template <>
struct Mfma<F16> {
  static __device__ __forceinline__ f4_t qk(u32x4 a, u32x4 b, f4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, a), __builtin_bit_cast(h8_t, b), c,
                                                  0, 0, 0);
  }
  static __device__ __forceinline__ f4_t pv(u32x2 a, u32x2 b, f4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h4_t, a), __builtin_bit_cast(h4_t, b), c,
                                                 0, 0, 0);
  }
  static constexpr uint32_t kOnes = 0x3C003C00u;  // two f16 1.0
  // two fp32 values -> one word of two f16 (round to nearest even)
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(lo))) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(hi))) << 16);
  }
};

template <>
struct Mfma<BF16> {
  static __device__ __forceinline__ f4_t qk(u32x4 a, u32x4 b, f4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8_t, a), __builtin_bit_cast(b8_t, b), c,
                                                   0, 0, 0);
  }
  static __device__ __forceinline__ f4_t pv(u32x2 a, u32x2 b, f4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4_t, a), __builtin_bit_cast(s4_t, b), c,
                                                     0, 0, 0);
  }
  static constexpr uint32_t kOnes = 0x3F803F80u;  // two bf16 1.0
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return static_cast<uint32_t>(BF16::pack(lo)) | (static_cast<uint32_t>(BF16::pack(hi)) << 16);
  }
};

// One operand word of V^T: element e (< 4) of slice a in the low half and
// element e of slice b in the high half (one v_perm_b32: result bytes pick
// bytes of wa (selector values 0-3) and wb (4-7)).
__device__ __forceinline__ uint32_t col_pair(u32x2 a, u32x2 b, int e) {
  const uint32_t wa = (e < 2) ? a.x : a.y;
  const uint32_t wb = (e < 2) ? b.x : b.y;
  return __builtin_amdgcn_perm(wb, wa, (e & 1) ? 0x07060302u : 0x05040100u);
}

// Deferred rescaling: the running sums keep the reference max m until some
// row's scores exceed it by more than 2^kRescaleLog2 (then every row moves to
// its new max).  Until then probabilities are at most 2^kRescaleLog2 = 256,
// well inside fp32 and the 16-bit types the P.V products take; the final
// ratio sum / weight does not depend on the reference, so only the number of
// rescalings changes (rare after the first chunks of a row).
constexpr float kRescaleLog2 = 8.f;

// Operand words of the P.V products.  With KB = 2 key blocks of 16 per chunk
// the product is 16x16x32 and its K index 8*(l/16) + j of lane l stands for
// key 4*(l/16) + j (j < 4) of block 0 and key 16 + 4*(l/16) + j - 4 of block
// 1 — any labelling of the summed index works as long as both operands use
// it; with KB = 1 it is 16x16x16 over keys 4*(l/16) + j.
template <typename T, int KB>
struct PvOps;

template <typename T>
struct PvOps<T, 1> {
  using word_t = u32x2;
  static __device__ __forceinline__ f4_t mma(word_t a, word_t b, f4_t c) { return Mfma<T>::pv(a, b, c); }
};

template <>
struct PvOps<F16, 2> {
  using word_t = u32x4;
  static __device__ __forceinline__ f4_t mma(word_t a, word_t b, f4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, a), __builtin_bit_cast(h8_t, b), c,
                                                  0, 0, 0);
  }
};

template <>
struct PvOps<BF16, 2> {
  using word_t = u32x4;
  static __device__ __forceinline__ f4_t mma(word_t a, word_t b, f4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8_t, a), __builtin_bit_cast(b8_t, b), c,
                                                   0, 0, 0);
  }
};

}  // namespace pa
