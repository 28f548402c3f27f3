// Matrix-core (MFMA) operand helpers shared by the query kernels
// (pa_prefill.hip) and the grouped-query decode kernel (pa_decode_mfma.hip),
// gfx950: the 16x16x32 / 16x16x16 fp16 and bf16 products, the operand words
// of the P.V product and the deferred-rescaling bound.
#pragma once

#include "pa_device.h"
#include "pa_attend.h"

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

// Log-sum-exp merge of rows split into several partitions, a kernel of its
// own (after the kernel that wrote the partials): one workgroup per
// (sequence, query head, SLICE-element slice of the D output elements).
// Partials are laid out by item — (sequence, head group, partition), the
// partition fastest — with `group` heads per item: the partial of head h of
// sequence s in partition p sits in slot (off[s] + (h / group) * parts + p)
// * group + h % group, where off[] (S + 1 item offsets) and the partition
// size P (off[S + 1]) are what the first kernel wrote.  A row of one
// partition was written by the first kernel: nothing to do.  A partial is
// o_p = acc_p / l_p in the 16-bit type (D elements per slot) with (m_p, l_p)
// in fp32, and weighs l_p 2^(m_p - M).  kC = SLICE / 4
// lanes cover one partial's slice (4 values each) and the kG lane groups take
// every kG-th partial, kU per round with all their loads issued at once;
// each round is folded into a running (max, sum, sums) with the online
// rescaling, and the groups are combined through LDS.
template <typename T, int D, int SLICE, int THREADS>
__global__ __launch_bounds__(THREADS) void lse_merge_kernel(
    typename T::storage* __restrict__ out, const int* __restrict__ ws_off, const float* __restrict__ ws_ml,
    const float* __restrict__ ws_acc, const int32_t* __restrict__ context_lens, int num_seqs, int num_heads,
    int group, int cap) {
  static_assert(D % SLICE == 0 && SLICE % 4 == 0 && THREADS % (SLICE / 4) == 0, "whole slices");
  constexpr int kSlices = D / SLICE;
  constexpr int kC = SLICE / 4;
  constexpr int kG = THREADS / kC;
  constexpr int kU = 8;
  __shared__ float s_M[kG];
  __shared__ float s_den[kG];
  __shared__ f4_t s_num[kG][kC];
  const int slice = blockIdx.x % kSlices;
  const int row = blockIdx.x / kSlices;
  const int s = row / num_heads;
  const int h = row % num_heads;
  const int L = min(max(context_lens[s], 0), cap);
  const int P = ws_off[num_seqs + 1];
  const int parts = (L + P - 1) / P;
  if (parts <= 1) return;
  const size_t item0 = static_cast<size_t>(ws_off[s]) + static_cast<size_t>(h / group) * parts;
  const int g = h % group;
  const int tid = threadIdx.x;
  const int c = tid % kC;
  const int grp = tid / kC;
  const int e0 = slice * SLICE + 4 * c;  // first element of this lane
  float Mx = -INFINITY, den = 0.f;
  f4_t num = {0.f, 0.f, 0.f, 0.f};
  for (int p0 = grp; p0 < parts; p0 += kG * kU) {
    f32x2 ml[kU];
    f4_t v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const size_t slot = (item0 + min(p0 + u * kG, parts - 1)) * group + g;
      ml[u] = *reinterpret_cast<const f32x2*>(ws_ml + slot * 2);
      const u32x2 w = *reinterpret_cast<const u32x2*>(
          reinterpret_cast<const typename T::storage*>(ws_acc) + slot * D + e0);
      float f[4];
      T::unpack_word(w.x, f);
      T::unpack_word(w.y, f + 2);
      v[u] = f4_t{f[0], f[1], f[2], f[3]};
    }
    float bm = -INFINITY;
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (p0 + u * kG < parts) bm = fmaxf(bm, ml[u][0]);
    const float mn = fmaxf(Mx, bm);
    if (mn == -INFINITY) continue;  // only empty partials so far
    const float a = (Mx == -INFINITY) ? 0.f : fast_exp2(Mx - mn);
    den *= a;
    num *= a;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const float mu = ml[u][0];
      // partial p holds o_p = acc_p / l_p: it weighs l_p 2^(m_p - M)
      const float wl = ((p0 + u * kG < parts && mu != -INFINITY) ? fast_exp2(mu - mn) : 0.f) * ml[u][1];
      den += wl;
      num += wl * v[u];
    }
    Mx = mn;
  }
  if (kG == 1) {  // one lane group: nothing to combine
    const float inv = 1.f / den;
    const uint32_t w0 = Mfma<T>::pack2(num[0] * inv, num[1] * inv);
    const uint32_t w1 = Mfma<T>::pack2(num[2] * inv, num[3] * inv);
    *reinterpret_cast<u32x2*>(out + (static_cast<size_t>(s) * num_heads + h) * D + e0) = u32x2{w0, w1};
    return;
  }
  if (c == 0) {
    s_M[grp] = Mx;
    s_den[grp] = den;
  }
  s_num[grp][c] = num;
  __syncthreads();
  if (tid >= kC) return;
  float M2 = -INFINITY;
#pragma unroll
  for (int k = 0; k < kG; ++k) M2 = fmaxf(M2, s_M[k]);
  float d = 0.f;
  f4_t o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int k = 0; k < kG; ++k) {
    const float f = (s_M[k] == -INFINITY) ? 0.f : fast_exp2(s_M[k] - M2);
    d = fmaf(f, s_den[k], d);
    o += f * s_num[k][tid];
  }
  const float inv = 1.f / d;
  const uint32_t w0 = Mfma<T>::pack2(o[0] * inv, o[1] * inv);
  const uint32_t w1 = Mfma<T>::pack2(o[2] * inv, o[3] * inv);
  *reinterpret_cast<u32x2*>(out + (static_cast<size_t>(s) * num_heads + h) * D + e0) = u32x2{w0, w1};
}

}  // namespace pa
