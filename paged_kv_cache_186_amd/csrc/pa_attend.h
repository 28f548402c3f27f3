// Shared pieces of the decode kernels (gfx950): tile geometry, the per-tile
// online-softmax update, log-sum-exp combination and coherent accesses to the
// workspace.
#pragma once

#include "pa_device.h"

namespace pa {

constexpr float kLog2e = 1.4426950408889634f;

template <typename T, int D, int BS>
struct Tile {
  static constexpr int kElems = T::kElems;                       // per 16-byte vector
  static constexpr int kLanesPerRow = D / kElems;                // 8, 16 or 32
  static constexpr int kRowsPerLoad = kWave / kLanesPerRow;      // 8, 4 or 2
  static constexpr int kLoads = BS / kRowsPerLoad;               // per tensor per tile
  static constexpr int kRowBytes = D * static_cast<int>(sizeof(typename T::storage));
  static constexpr int kTileBytes = BS * kRowBytes;
  static constexpr int kLoadBytes = kWave * kVecBytes;           // 1 KiB per wave instruction
  static_assert(kLanesPerRow * kVecBytes == kRowBytes, "a row is a whole number of lane vectors");
  static_assert(kLoads * kLoadBytes == kTileBytes, "a tile is a whole number of wave loads");
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Online-softmax update of one lane group with one loaded tile.  kMasked
// handles the last, partly filled block: rows at or past L get weight exactly
// 0 and their V values are replaced by 0 (they may hold NaN).  For a scaled
// (8-bit) KV type, sk and sv are the tile's K and V scales: scores are
// sk * <q, k_code> and V rows enter as sv * v_code (sv is folded into the
// weight of the V sum, not into l).  All 64 lanes must be active (the DPP
// sums read every lane).
template <typename T, int D, int BS, bool kMasked>
__device__ __forceinline__ void attend_tile(const u32x4 (&kv)[Tile<T, D, BS>::kLoads],
                                            const u32x4 (&vv)[Tile<T, D, BS>::kLoads],
                                            const float (&qf)[T::kElems], float& m, float& l,
                                            float (&acc)[T::kElems], int tok0, int L,
                                            float sk = 1.f, float sv = 1.f) {
  using C = Tile<T, D, BS>;
  float sc[C::kLoads];
#pragma unroll
  for (int i = 0; i < C::kLoads; ++i) {
    float kf[T::kElems];
    T::unpack(kv[i], kf);
    float d = 0.f;
#pragma unroll
    for (int e = 0; e < T::kElems; ++e) d = fmaf(qf[e], kf[e], d);
    sc[i] = group_sum<C::kLanesPerRow>(d);
    if constexpr (T::kScaled) sc[i] *= sk;
  }

  bool ok[C::kLoads];
  float bm = -INFINITY;
#pragma unroll
  for (int i = 0; i < C::kLoads; ++i) {
    ok[i] = !kMasked || (tok0 + i * C::kRowsPerLoad < L);
    if (ok[i]) bm = fmaxf(bm, sc[i]);
  }
  const float mn = fmaxf(m, bm);
  // mn is -inf only while this group has met no token: nothing to rescale then.
  const float alpha = (mn == -INFINITY) ? 1.f : fast_exp2(m - mn);
  l *= alpha;
#pragma unroll
  for (int e = 0; e < T::kElems; ++e) acc[e] *= alpha;
  // Branch-free on purpose: rows past L are selected to weight 0 and value 0
  // (never 0 * NaN), and every loaded register is read on every path, which
  // lets the compiler keep the next tile's loads in flight across this call.
#pragma unroll
  for (int i = 0; i < C::kLoads; ++i) {
    const float p = ok[i] ? fast_exp2(sc[i] - mn) : 0.f;
    float vf[T::kElems];
    T::unpack(vv[i], vf);
    l += p;
    float pv = p;
    if constexpr (T::kScaled) pv *= sv;
#pragma unroll
    for (int e = 0; e < T::kElems; ++e) acc[e] = fmaf(pv, ok[i] ? vf[e] : 0.f, acc[e]);
  }
  m = mn;
}

// attend_tile for GW query heads that share one K/V tile (grouped-query
// attention): every K and V vector is loaded once and serves all GW heads'
// dot products, online softmax updates and weighted V sums.  This is where the
// per-byte arithmetic grows GW-fold, so it is kept lean:
//  * 16-bit caches (T::kDot2) take the scores with v_dot2 on the packed
//    words of K and of the query (qw: the query's own 16-bit words, unscaled;
//    qscale is applied to each score), with no unpacking of K;
//  * the running sums are rescaled only when some lane's maximum grew (a
//    wave-uniform test; after the first tiles of a row it rarely does).
template <typename T, int D, int BS, int GW, bool kMasked>
__device__ __forceinline__ void attend_tile_heads(const u32x4 (&kv)[Tile<T, D, BS>::kLoads],
                                                  const u32x4 (&vv)[Tile<T, D, BS>::kLoads],
                                                  const float (&qf)[GW][T::kElems],
                                                  const uint32_t (&qw)[GW][T::kElems / 2], float qscale,
                                                  float (&m)[GW], float (&l)[GW],
                                                  float (&acc)[GW][T::kElems], int tok0, int L, float sk,
                                                  float sv) {
  using C = Tile<T, D, BS>;
  float sc[GW][C::kLoads];
#pragma unroll
  for (int i = 0; i < C::kLoads; ++i) {
    if constexpr (T::kDot2) {
      const uint32_t kw[4] = {kv[i].x, kv[i].y, kv[i].z, kv[i].w};
#pragma unroll
      for (int g = 0; g < GW; ++g) {
        float d = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) d = T::dot2(qw[g][w], kw[w], d);
        sc[g][i] = group_sum<C::kLanesPerRow>(d) * qscale;
      }
    } else {
      float kf[T::kElems];
      T::unpack(kv[i], kf);
#pragma unroll
      for (int g = 0; g < GW; ++g) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < T::kElems; ++e) d = fmaf(qf[g][e], kf[e], d);
        sc[g][i] = group_sum<C::kLanesPerRow>(d);
        if constexpr (T::kScaled) sc[g][i] *= sk;
      }
    }
  }
  bool ok[C::kLoads];
#pragma unroll
  for (int i = 0; i < C::kLoads; ++i) ok[i] = !kMasked || (tok0 + i * C::kRowsPerLoad < L);
  float p[GW][C::kLoads];
#pragma unroll
  for (int g = 0; g < GW; ++g) {
    float bm = -INFINITY;
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i)
      if (ok[i]) bm = fmaxf(bm, sc[g][i]);
    const float mn = fmaxf(m[g], bm);
    if (__builtin_amdgcn_ballot_w64(mn > m[g]) != 0) {  // some lane's maximum grew
      // mn is -inf only while a group has met no token: nothing to rescale then
      const float alpha = (mn == -INFINITY) ? 1.f : fast_exp2(m[g] - mn);
      l[g] *= alpha;
#pragma unroll
      for (int e = 0; e < T::kElems; ++e) acc[g][e] *= alpha;
      m[g] = mn;
    }
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) p[g][i] = ok[i] ? fast_exp2(sc[g][i] - m[g]) : 0.f;
  }
  if constexpr (__is_same(T, F16) && C::kLoads % 2 == 0) {
    // fp16 cache: the weighted sums by packed dot products over PAIRS of
    // rows — loads i and i+1 hold rows 4 apart in the same lanes, so byte
    // permutes turn their words into (row i, row i+1) pairs per element, and
    // each head's two weights are rounded to fp16 (relative error <= 2^-11)
    // into one word: half the multiply-adds of the per-row form.  The row
    // sums take the same rounded weights (a dot product with (1, 1)).  A
    // bf16 cache keeps the fp32 weights (bf16 would round them to 2^-8).
#pragma unroll
    for (int i = 0; i < C::kLoads; i += 2) {
      uint32_t a[4] = {vv[i].x, vv[i].y, vv[i].z, vv[i].w};
      uint32_t b[4] = {vv[i + 1].x, vv[i + 1].y, vv[i + 1].z, vv[i + 1].w};
      if constexpr (kMasked) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          a[w] = ok[i] ? a[w] : 0u;
          b[w] = ok[i + 1] ? b[w] : 0u;
        }
      }
      uint32_t lo[4], hi[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        lo[w] = __builtin_amdgcn_perm(b[w], a[w], 0x05040100u);  // element 2w of both rows
        hi[w] = __builtin_amdgcn_perm(b[w], a[w], 0x07060302u);  // element 2w + 1
      }
#pragma unroll
      for (int g = 0; g < GW; ++g) {
        const uint32_t pp = T::pack_pair(p[g][i], p[g][i + 1]);
        l[g] = T::dot2(pp, T::kOnePair, l[g]);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          acc[g][2 * w] = T::dot2(pp, lo[w], acc[g][2 * w]);
          acc[g][2 * w + 1] = T::dot2(pp, hi[w], acc[g][2 * w + 1]);
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      float vf[T::kElems];
      T::unpack(vv[i], vf);
#pragma unroll
      for (int e = 0; e < T::kElems; ++e) vf[e] = ok[i] ? vf[e] : 0.f;
#pragma unroll
      for (int g = 0; g < GW; ++g) {
        l[g] += p[g][i];
        float pv = p[g][i];
        if constexpr (T::kScaled) pv *= sv;
#pragma unroll
        for (int e = 0; e < T::kElems; ++e) acc[g][e] = fmaf(pv, vf[e], acc[g][e]);
      }
    }
  }
}

// The query / output side of a lane: E = KT::kElems consecutive elements of a
// row, stored as QT — one 16-byte vector when QT and KT have the same width,
// two for an 8-bit KV cache read with a 16-bit query.
template <typename QT, typename KT>
struct QSlice {
  static constexpr int kElems = KT::kElems;
  static constexpr int kBytes = kElems * static_cast<int>(sizeof(typename QT::storage));
  static constexpr int kVecs = kBytes / kVecBytes;
  static_assert(kVecs * kVecBytes == kBytes && kVecs * QT::kElems == kElems, "whole vectors");

  // fp32 values of the lane's slice of one row (row points at element 0)
  static __device__ __forceinline__ void load(const typename QT::storage* row, int col, float* f) {
    const char* p = reinterpret_cast<const char*>(row) + col * kBytes;
#pragma unroll
    for (int i = 0; i < kVecs; ++i) QT::unpack(load16(p + i * kVecBytes), f + i * QT::kElems);
  }
  // round the lane's slice to QT and store it
  static __device__ __forceinline__ void store(typename QT::storage* row, int col, const float* f) {
    char* p = reinterpret_cast<char*>(row) + col * kBytes;
#pragma unroll
    for (int i = 0; i < kVecs; ++i) {
      typename QT::storage s[QT::kElems];
#pragma unroll
      for (int e = 0; e < QT::kElems; ++e) s[e] = QT::pack(f[i * QT::kElems + e]);
      u32x4 w;
      static_assert(sizeof(s) == sizeof(w), "16-byte slice");
      __builtin_memcpy(&w, s, sizeof(w));
      store16(p + i * kVecBytes, w);
    }
  }
};

// Workspace accesses shared between workgroups on different XCDs use
// agent-scope relaxed atomics: on gfx950 these are L2-bypassing (sc1) loads
// and stores, coherent across XCDs without any cache write-back or invalidate.
__device__ __forceinline__ uint64_t load_coherent_u64(const float* p) {
  return __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// (m, d) <- lse-combine of (m, d) and (m2, d2); empty states have m = -inf.
__device__ __forceinline__ void lse_combine(float& m, float& d, float m2, float d2) {
  if (m2 == -INFINITY) return;
  if (m == -INFINITY) {
    m = m2;
    d = d2;
    return;
  }
  const float mn = fmaxf(m, m2);
  d = d * fast_exp2(m - mn) + d2 * fast_exp2(m2 - mn);
  m = mn;
}

__device__ __forceinline__ void store_coherent_u64(float* p, float lo, float hi) {
  const uint64_t v = static_cast<uint64_t>(__builtin_bit_cast(uint32_t, lo)) |
                     (static_cast<uint64_t>(__builtin_bit_cast(uint32_t, hi)) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float lo_float(uint64_t v) { return __builtin_bit_cast(float, static_cast<uint32_t>(v)); }
__device__ __forceinline__ float hi_float(uint64_t v) { return __builtin_bit_cast(float, static_cast<uint32_t>(v >> 32)); }

}  // namespace pa
