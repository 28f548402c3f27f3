// Device-side building blocks shared by the libpagedattn kernels (gfx950).
//
// Storage types are tag structs that know how to turn one 16-byte vector
// (what one lane moves with a global_load_dwordx4) into fp32 values and how to
// round an fp32 result back to storage with round-to-nearest-even.  The 8-bit
// KV-cache types (FP8E4M3, FP8E5M2) only unpack; their values are scaled per
// (block, head) (kScaled) and written by the quantizers at the end.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kVecBytes = 16;

// Reinterpret one 32-bit word as fp32.  The word is taken by value on
// purpose: this clang lowers __builtin_bit_cast applied directly to an
// ext-vector element (v.y, v.z, ...) as a cast of the vector's FIRST word.
__device__ __forceinline__ float word_as_float(uint32_t w) { return __builtin_bit_cast(float, w); }

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// kDot2: the type has a two-element dot product with fp32 accumulation
// (v_dot2_f32_f16 / _bf16), dot2(a, b, c) = a.x*b.x + a.y*b.y + c, on packed
// 32-bit words of two elements each.
struct F32 {
  using storage = float;
  static constexpr int kElems = 4;  // per 16-byte vector
  static constexpr bool kScaled = false;
  static constexpr bool kDot2 = false;
  static __device__ __forceinline__ void unpack(const u32x4 v, float* f) {
    const uint32_t w0 = v.x, w1 = v.y, w2 = v.z, w3 = v.w;
    f[0] = word_as_float(w0);
    f[1] = word_as_float(w1);
    f[2] = word_as_float(w2);
    f[3] = word_as_float(w3);
  }
  static __device__ __forceinline__ storage pack(float x) { return x; }
};

struct F16 {
  using storage = _Float16;
  static constexpr int kElems = 8;
  static constexpr bool kScaled = false;
  static constexpr bool kDot2 = true;
  static constexpr uint32_t kOnePair = 0x3C003C00u;  // (1.0, 1.0)
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c, false);
  }
  static __device__ __forceinline__ void unpack_word(uint32_t w, float* f) {
    const f16x2 h = __builtin_bit_cast(f16x2, w);
    f[0] = static_cast<float>(h.x);
    f[1] = static_cast<float>(h.y);
  }
  static __device__ __forceinline__ void unpack(const u32x4 v, float* f) {
    unpack_word(v.x, f + 0);
    unpack_word(v.y, f + 2);
    unpack_word(v.z, f + 4);
    unpack_word(v.w, f + 6);
  }
  // v_cvt_f16_f32 rounds to nearest even in the default rounding mode.
  static __device__ __forceinline__ storage pack(float x) { return static_cast<_Float16>(x); }
  // two fp32 values -> one word of two (round to nearest even)
  static __device__ __forceinline__ uint32_t pack_pair(float lo, float hi) {
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, pack(lo))) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, pack(hi))) << 16);
  }
};

struct BF16 {
  using storage = uint16_t;
  static constexpr int kElems = 8;
  static constexpr bool kScaled = false;
  static constexpr bool kDot2 = true;
  static constexpr uint32_t kOnePair = 0x3F803F80u;  // (1.0, 1.0)
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
  }
  static __device__ __forceinline__ void unpack_word(uint32_t w, float* f) {
    f[0] = __builtin_bit_cast(float, w << 16);
    f[1] = __builtin_bit_cast(float, w & 0xffff0000u);
  }
  static __device__ __forceinline__ void unpack(const u32x4 v, float* f) {
    unpack_word(v.x, f + 0);
    unpack_word(v.y, f + 2);
    unpack_word(v.z, f + 4);
    unpack_word(v.w, f + 6);
  }
  // fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.
  static __device__ __forceinline__ storage pack(float x) {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
  }
  static __device__ __forceinline__ uint32_t pack_pair(float lo, float hi) {
    return static_cast<uint32_t>(pack(lo)) | (static_cast<uint32_t>(pack(hi)) << 16);
  }
};

// 8-bit floating-point KV elements, OCP formats: E4M3 (bias 7, no
// infinities, S.1111.111 = NaN, largest finite 448) and E5M2 (bias 15,
// IEEE-style infinities and NaNs, largest finite 57344).  gfx950's
// v_cvt_pk_f32_fp8 / _bf8 decode two codes of one 32-bit word per
// instruction in these formats.
typedef float f32x2 __attribute__((ext_vector_type(2)));

struct FP8E4M3 {
  using storage = uint8_t;
  static constexpr int kElems = 16;
  static constexpr bool kScaled = true;
  static constexpr bool kDot2 = false;
  static __device__ __forceinline__ void unpack_word(uint32_t w, float* f) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
    f[0] = lo.x;
    f[1] = lo.y;
    f[2] = hi.x;
    f[3] = hi.y;
  }
  static __device__ __forceinline__ void unpack(const u32x4 v, float* f) {
    unpack_word(v.x, f + 0);
    unpack_word(v.y, f + 4);
    unpack_word(v.z, f + 8);
    unpack_word(v.w, f + 12);
  }
};

struct FP8E5M2 {
  using storage = uint8_t;
  static constexpr int kElems = 16;
  static constexpr bool kScaled = true;
  static constexpr bool kDot2 = false;
  static __device__ __forceinline__ void unpack_word(uint32_t w, float* f) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_bf8(static_cast<int>(w), false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_bf8(static_cast<int>(w), true);
    f[0] = lo.x;
    f[1] = lo.y;
    f[2] = hi.x;
    f[3] = hi.y;
  }
  static __device__ __forceinline__ void unpack(const u32x4 v, float* f) {
    unpack_word(v.x, f + 0);
    unpack_word(v.y, f + 4);
    unpack_word(v.z, f + 8);
    unpack_word(v.w, f + 12);
  }
};

// fp32 -> 8-bit code: nearest value, ties to the even code, saturating to the
// largest finite value (infinities included), NaN -> 0x7F; the sign bit is
// y's (so -0 -> 0x80).  Normal results keep the top kMant mantissa bits of
// y, rounded to nearest even on the fp32 bit pattern (a carry into the
// exponent field is the correct next binade); subnormal results are
// rint(|y| * 2^(bias - 1 + kMant)), exact because that scaling is a power of
// two, and the rounding of the largest subnormal up to the smallest normal
// lands on the smallest normal's code.
template <int kExp, int kMant, int kBias>
__device__ __forceinline__ uint32_t quantize_fp8(float y, float max_finite, uint32_t max_code) {
  const uint32_t u = __builtin_bit_cast(uint32_t, y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;                                    // NaN
  if (__builtin_bit_cast(float, a) >= max_finite) return sign | max_code;  // saturate
  constexpr float kMinNormal = __builtin_bit_cast(float, static_cast<uint32_t>(127 + 1 - kBias) << 23);
  constexpr float kSubScale = __builtin_bit_cast(float, static_cast<uint32_t>(127 + kBias - 1 + kMant) << 23);
  uint32_t code;
  if (__builtin_bit_cast(float, a) < kMinNormal) {
    code = static_cast<uint32_t>(__builtin_rintf(__builtin_bit_cast(float, a) * kSubScale));
  } else {
    constexpr int kDrop = 23 - kMant;
    const uint32_t r = (a + ((1u << (kDrop - 1)) - 1u) + ((a >> kDrop) & 1u)) >> kDrop;
    code = r - (static_cast<uint32_t>(127 - kBias) << kMant);
  }
  return sign | code;
}

__device__ __forceinline__ uint32_t quantize_e4m3(float y) { return quantize_fp8<4, 3, 7>(y, 448.f, 0x7eu); }
__device__ __forceinline__ uint32_t quantize_e5m2(float y) { return quantize_fp8<5, 2, 15>(y, 57344.f, 0x7bu); }

// ---------------------------------------------------------------------------
// Cross-lane sums over aligned groups of G consecutive lanes (G = 4 ... 32),
// leaving the group total in every lane of the group.  DPP quad permutes give
// the xor-1 and xor-2 partners; row_half_mirror (lane i <- 7-i within 8) and
// row_mirror (lane i <- 15-i within 16) then pair each lane with one in the
// other half, which completes the 8- and 16-lane sums; ds_swizzle with xor
// mask 16 crosses the two rows of a 32-lane half-wave.  Every source lane of
// these permutations is a valid lane of the same row and the sums run with
// the whole wave active, so the bound-control bit (a zero source for invalid
// or inactive lanes) never takes effect; setting it lets the compiler fold
// each move into the following add (one DPP add per step).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float dpp_quad_xor1(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_quad_xor2(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_row_half_mirror(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_row_mirror(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x140, 0xF, 0xF, true));
}

// Exchanges between lane groups without the LDS crossbar (__shfl_xor becomes
// ds_bpermute, an LDS round trip of ~100+ cycles per value).
//  * row_ror<N>: each lane reads lane (i - N) mod 16 of its 16-lane row (DPP);
//  * swap_pair<16> / swap_pair<32>: v_permlane16_swap (v_permlane32_swap),
//    given x in both operands, leaves x of the lower lane of each pair
//    (l, l ^ 16) (or (l, l ^ 32)) in the first register and x of the upper
//    lane in the second, in both lanes of the pair, so sums and maxima of the
//    two end with the same bits in both lanes.
template <int N>
__device__ __forceinline__ float row_ror(float x) {
  static_assert(N == 4 || N == 8, "rotations by 4 or 8 lanes");
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x120 + N, 0xF, 0xF, true));
}
template <int OFF>
__device__ __forceinline__ void swap_pair(float x, float& lo, float& hi) {
  static_assert(OFF == 16 || OFF == 32, "lane swaps across 16 or 32 lanes");
  // Written out: this compiler's __builtin_amdgcn_permlane{16,32}_swap hands
  // back the first register of the pair in both result elements.  b is a copy
  // of x; the two wait states cover the VALU writes of both operands before
  // the swap reads them (as the compiler itself places them).
  uint32_t a = __builtin_bit_cast(uint32_t, x);
  uint32_t b;
  if constexpr (OFF == 16)
    asm("v_mov_b32 %1, %0\n\ts_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "=&v"(b));
  else
    asm("v_mov_b32 %1, %0\n\ts_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "=&v"(b));
  lo = __builtin_bit_cast(float, a);
  hi = __builtin_bit_cast(float, b);
}

// ceil(x / d) for 0 <= x < 2^31 and 0 < d < 2^20, given rd = 1.0 / d in
// double precision: the product's relative error (below 2^-52) can only
// take an exact quotient k to just under k, so the truncated estimate is
// floor(x / d) or one less, and one remainder test corrects it.
__device__ __forceinline__ int ceil_div_nonneg(int x, int d, double rd) {
  int q = static_cast<int>(static_cast<double>(x) * rd);
  int r = x - q * d;
  if (r >= d) {
    ++q;
    r -= d;
  }
  return q + (r > 0 ? 1 : 0);
}

// Logical index of workgroup b of a G-workgroup grid such that consecutive
// logical indices run on one XCD: the dispatcher deals workgroups to the 8
// XCDs in turn (b goes to XCD b % 8), so XCD x holds the x-th contiguous
// range of logical indices (G / 8 of them, one more for the first G % 8).
__device__ __forceinline__ int xcd_local_index(int b, int G) {
  const int x = b & 7;
  return x * (G >> 3) + min(x, G & 7) + (b >> 3);
}

// Inclusive prefix sum of x over the 64 lanes of a wave, in DPP steps (no
// LDS round trips): sums within each 16-lane row by shifts of 1, 2, 4 and 8
// lanes (a lane shifted in from outside the row reads 0), then the total of
// row 0 added to row 1 and of row 2 to row 3 (row_bcast:15, rows 1 and 3
// written), then the total of rows 0-1 to rows 2 and 3 (row_bcast:31).  All
// 64 lanes must be active.
__device__ __forceinline__ int wave_prefix_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return x;
}

// Sum / maximum of x over the lanes that share lane % G (G = 4, 8, 16 or 32):
// the lane groups of a wave folded into one.  The maximum is the same in
// every lane; the sum is complete in every lane (for G >= 8 also bit-identical
// across lanes; for G = 4 the first two steps associate differently per lane).
template <int G>
__device__ __forceinline__ float fold_sum(float x) {
  static_assert(G == 4 || G == 8 || G == 16 || G == 32, "fold over groups of 4, 8, 16 or 32 lanes");
  if constexpr (G == 4) x += row_ror<4>(x);
  if constexpr (G <= 8) x += row_ror<8>(x);
  float lo, hi;
  if constexpr (G <= 16) {
    swap_pair<16>(x, lo, hi);
    x = lo + hi;
  }
  swap_pair<32>(x, lo, hi);
  return lo + hi;
}
template <int G>
__device__ __forceinline__ float fold_max(float x) {
  static_assert(G == 4 || G == 8 || G == 16 || G == 32, "fold over groups of 4, 8, 16 or 32 lanes");
  if constexpr (G == 4) x = fmaxf(x, row_ror<4>(x));
  if constexpr (G <= 8) x = fmaxf(x, row_ror<8>(x));
  float lo, hi;
  if constexpr (G <= 16) {
    swap_pair<16>(x, lo, hi);
    x = fmaxf(lo, hi);
  }
  swap_pair<32>(x, lo, hi);
  return fmaxf(lo, hi);
}

template <int G>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(G == 4 || G == 8 || G == 16 || G == 32, "group of 4, 8, 16 or 32 lanes");
  x += dpp_quad_xor1(x);
  x += dpp_quad_xor2(x);
  if constexpr (G >= 8) x += dpp_row_half_mirror(x);
  if constexpr (G >= 16) x += dpp_row_mirror(x);
  if constexpr (G >= 32) {
    float lo, hi;
    swap_pair<16>(x, lo, hi);
    x = lo + hi;
  }
  return x;
}

// Word 3 of a gfx9-family buffer resource for raw (unformatted, unswizzled)
// 32-bit accesses.
constexpr int kBufferRsrcWord3 = 0x00020000;

// One fp32 read from a wave-uniform address through the VECTOR memory path
// (a 4-byte buffer resource at p).  The compiler would turn a plain uniform
// load into a scalar load, and it waits for all outstanding scalar loads at
// once; for per-tile scales that stalled every pipeline stage on the previous
// tile's scale.  A vector load completes in order with the tile's own loads.
__device__ __forceinline__ float load_uniform_f32(const float* p) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p), 0, sizeof(float), kBufferRsrcWord3);
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, 0, 0, 0));
}

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// K/V cache reads of the decode kernels: every byte is used once per call, so
// they are non-temporal (streaming) loads, which keep the stream from
// displacing other lines in the caches.  Measured against plain loads on the
// same kernels: 4 x 131072 tokens 1399 -> 1240 us, 131072 tokens 355 -> 318
// us, continuous batching 154 -> 136 us, layer shape 24.2 -> 22.2 us; the
// grouped-query matrix-core kernel 55.7 -> 49.2 us (4 K/V heads over 128K).
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x2_t load8_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
}
__device__ __forceinline__ void store16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

}  // namespace pa
