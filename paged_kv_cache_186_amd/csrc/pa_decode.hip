// Paged decode attention kernels for gfx950.
//
// What is computed: for each sequence s and head h, single-query softmax
// attention over the first L_s cached tokens, whose K/V rows are found through
// the block table (row t % BS of physical block table[s][t / BS]).  Sources:
// page "PagedAttentionMetal：基于Metal 3的Apple Silicon原生LLM推理加速方案",
// section 注意力计算优化 (fetch K/V via block-table lookups, no padding across a
// variable-length batch); vLLM tutorial page "3. PagedAttention原理", §3.2 and
// the closing remarks of §3.4 (paging leaves the attention arithmetic as is).
// Long contexts are cut into partitions whose softmax partials are merged with
// the log-sum-exp identity, the split-context decode the page "PagedAttention
// MLX：为Apple Silicon打造的高吞吐量LLM推理引擎" names ("Flash-Dec", roadmap
// milestone 4) without describing.
//
// How (our design, not the pages'): decode is a matrix-vector product per
// (sequence, head), so it is HBM-bound and MFMA would idle; the kernels are
// built around streaming each (block, head) tile — BS*D contiguous elements,
// 4 KiB for fp16 D=128 BS=16 — with every lane moving 16 bytes per load, so one
// wave instruction covers 1 KiB of contiguous memory.
//
// Lane layout inside one wave for one tile: a cache row of D elements is spread
// over LPR = D*elem/16 consecutive lanes, so one load instruction covers
// RPL = 64/LPR rows and a tile takes BS/RPL loads per tensor.  Each aligned
// group of LPR lanes keeps its OWN online-softmax state (running max m,
// running sum l, and the lane's slice of the weighted V sum), so the hot loop
// needs only the in-group dot-product reduction (DPP) and no cross-group or
// cross-wave traffic; the RPL*NW group states of a workgroup are merged once,
// through LDS, at the end.  Scores are kept in base-2 units (q is pre-scaled by
// scale*log2(e)) so every exponential is a single v_exp_f32.

#include "pa_device.h"
#include "pa_internal.h"
#include "pagedattn.h"

namespace pa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWavesPerGroup = 4;  // waves per workgroup of the partition kernel

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

// One (block, head) tile: scores for this lane-group's rows, online-softmax
// update, weighted V accumulation.  kMasked handles the last, partly filled
// block: rows at or past L get weight exactly 0 and their V is never touched
// (they may hold NaN).  All 64 lanes must be active (the DPP sums read every lane).
template <typename T, int D, int BS, bool kMasked>
__device__ __forceinline__ void attend_tile(const char* __restrict__ kb, const char* __restrict__ vb,
                                            const float (&qf)[T::kElems], float& m, float& l,
                                            float (&acc)[T::kElems], int lane, int tok0, int L) {
  using C = Tile<T, D, BS>;
  u32x4 kv[C::kLoads];
  u32x4 vv[C::kLoads];
#pragma unroll
  for (int i = 0; i < C::kLoads; ++i) kv[i] = load16(kb + i * C::kLoadBytes + lane * kVecBytes);
#pragma unroll
  for (int i = 0; i < C::kLoads; ++i) vv[i] = load16(vb + i * C::kLoadBytes + lane * kVecBytes);

  float sc[C::kLoads];
#pragma unroll
  for (int i = 0; i < C::kLoads; ++i) {
    float kf[T::kElems];
    T::unpack(kv[i], kf);
    float d = 0.f;
#pragma unroll
    for (int e = 0; e < T::kElems; ++e) d = fmaf(qf[e], kf[e], d);
    sc[i] = group_sum<C::kLanesPerRow>(d);
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
#pragma unroll
  for (int i = 0; i < C::kLoads; ++i) {
    if (ok[i]) {
      const float p = fast_exp2(sc[i] - mn);
      float vf[T::kElems];
      T::unpack(vv[i], vf);
      l += p;
#pragma unroll
      for (int e = 0; e < T::kElems; ++e) acc[e] = fmaf(p, vf[e], acc[e]);
    }
  }
  m = mn;
}

// Grid: (head, partition, sequence); NW waves per workgroup.  Workgroup
// (h, p, s) covers blocks [p*PB, min((p+1)*PB, nblk)) of sequence s; wave w
// takes blocks w, w+NW, ... of that range.  A sequence whose context fits one
// partition writes `out` directly; otherwise the partition's (max, sum) and
// unnormalised weighted V sum go to the workspace for decode_merge_kernel.
template <typename T, int D, int BS, int NW>
__global__ __launch_bounds__(NW* kWave) void decode_partition_kernel(
    typename T::storage* __restrict__ out, float* __restrict__ ws_ml, float* __restrict__ ws_acc,
    const typename T::storage* __restrict__ q, const char* __restrict__ k_pool,
    const char* __restrict__ v_pool, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, float q_scale, int num_heads, int num_blocks,
    int max_blocks, int part_blocks, int max_parts) {
  using C = Tile<T, D, BS>;
  constexpr int kGroups = NW * C::kRowsPerLoad;
  __shared__ float s_m[kGroups];
  __shared__ float s_l[kGroups];
  __shared__ float s_acc[kGroups][D];
  __shared__ int s_bad[NW];

  const int h = blockIdx.x;
  const int p = blockIdx.y;
  const int s = blockIdx.z;
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int L = min(max(context_lens[s], 0), max_blocks * BS);
  const int nblk = (L + BS - 1) / BS;
  const int nparts = (nblk + part_blocks - 1) / part_blocks;
  const size_t row = static_cast<size_t>(s) * num_heads + h;

  if (L == 0) {  // empty context: zero row (written once, by partition 0)
    if (p == 0)
      for (int d = threadIdx.x; d < D; d += blockDim.x) out[row * D + d] = T::pack(0.f);
    return;
  }
  if (p >= nparts) return;

  const int b_begin = p * part_blocks;
  const int b_end = min(nblk, b_begin + part_blocks);
  const int grp = lane / C::kLanesPerRow;
  const int col = lane % C::kLanesPerRow;

  float qf[T::kElems];
  T::unpack(load16(reinterpret_cast<const char*>(q + row * D) + col * kVecBytes), qf);
#pragma unroll
  for (int e = 0; e < T::kElems; ++e) qf[e] *= q_scale;

  float m = -INFINITY;
  float l = 0.f;
  float acc[T::kElems];
#pragma unroll
  for (int e = 0; e < T::kElems; ++e) acc[e] = 0.f;
  bool bad = false;

  const int32_t* tbl = block_tables + static_cast<size_t>(s) * max_blocks;
  for (int j = b_begin + wave; j < b_end; j += NW) {
    int phys = tbl[j];
    if (static_cast<unsigned>(phys) >= static_cast<unsigned>(num_blocks)) {
      bad = true;  // never dereference an id outside the pool
      phys = 0;
    }
    const size_t tile = (static_cast<size_t>(phys) * num_heads + h) * C::kTileBytes;
    const int tok0 = j * BS + grp;
    if ((j + 1) * BS <= L)
      attend_tile<T, D, BS, false>(k_pool + tile, v_pool + tile, qf, m, l, acc, lane, tok0, L);
    else
      attend_tile<T, D, BS, true>(k_pool + tile, v_pool + tile, qf, m, l, acc, lane, tok0, L);
  }

  // Merge the kGroups lane-group states of this workgroup through LDS.
  const int g = wave * C::kRowsPerLoad + grp;
  if (col == 0) {
    s_m[g] = m;
    s_l[g] = l;
  }
#pragma unroll
  for (int e = 0; e < T::kElems; ++e) s_acc[g][col * T::kElems + e] = acc[e];
  if (lane == 0) s_bad[wave] = bad ? 1 : 0;
  __syncthreads();

  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    int any_bad = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) any_bad |= s_bad[w];
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < kGroups; ++k) M = fmaxf(M, s_m[k]);
    float lsum = 0.f;
    float o = 0.f;
#pragma unroll
    for (int k = 0; k < kGroups; ++k) {
      const float a = fast_exp2(s_m[k] - M);  // groups that met no token: exp2(-inf) = 0
      lsum = fmaf(a, s_l[k], lsum);
      o = fmaf(a, s_acc[k][d], o);
    }
    if (any_bad) {
      o = __builtin_nanf("");
      lsum = __builtin_nanf("");
    }
    if (nparts == 1) {
      out[row * D + d] = T::pack(o / lsum);
    } else {
      const size_t prow = row * max_parts + p;
      ws_acc[prow * D + d] = o;
      if (d == 0) {
        ws_ml[prow * 2 + 0] = M;
        ws_ml[prow * 2 + 1] = lsum;
      }
    }
  }
}

// Log-sum-exp merge of the partitions of one (sequence, head): with M the
// largest partition max, out = sum_i 2^(m_i-M) acc_i / sum_i 2^(m_i-M) l_i.
// Grid (head, sequence), D threads; sequences with one partition are skipped
// (the partition kernel already wrote them).
template <typename T, int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(
    typename T::storage* __restrict__ out, const float* __restrict__ ws_ml,
    const float* __restrict__ ws_acc, const int32_t* __restrict__ context_lens, int num_heads,
    int block_size, int max_blocks, int part_blocks, int max_parts) {
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int d = threadIdx.x;
  const int L = min(max(context_lens[s], 0), max_blocks * block_size);
  const int nblk = (L + block_size - 1) / block_size;
  const int nparts = (nblk + part_blocks - 1) / part_blocks;
  if (nparts <= 1) return;
  const size_t row = static_cast<size_t>(s) * num_heads + h;
  const size_t base = row * max_parts;
  float M = -INFINITY;
  for (int i = 0; i < nparts; ++i) M = fmaxf(M, ws_ml[(base + i) * 2]);
  float num = 0.f;
  float den = 0.f;
  for (int i = 0; i < nparts; ++i) {
    const float a = fast_exp2(ws_ml[(base + i) * 2] - M);
    den = fmaf(a, ws_ml[(base + i) * 2 + 1], den);
    num = fmaf(a, ws_acc[(base + i) * D + d], num);
  }
  out[row * D + d] = T::pack(num / den);
}

template <typename T, int D, int BS>
hipError_t run_decode(const DecodeArgs& a, hipStream_t stream) {
  using S = typename T::storage;
  const dim3 grid(a.num_heads, a.max_partitions, a.num_seqs);
  hipLaunchKernelGGL((decode_partition_kernel<T, D, BS, kWavesPerGroup>), grid,
                     dim3(kWavesPerGroup * kWave), 0, stream, static_cast<S*>(a.out), a.ws_ml,
                     a.ws_acc, static_cast<const S*>(a.q), static_cast<const char*>(a.k_pool),
                     static_cast<const char*>(a.v_pool), a.block_tables, a.context_lens,
                     a.scale * kLog2e, a.num_heads, a.num_blocks, a.max_blocks_per_seq,
                     a.partition_blocks, a.max_partitions);
  if (a.max_partitions > 1) {
    hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3(a.num_heads, a.num_seqs), dim3(D), 0,
                       stream, static_cast<S*>(a.out), a.ws_ml, a.ws_acc, a.context_lens,
                       a.num_heads, BS, a.max_blocks_per_seq, a.partition_blocks,
                       a.max_partitions);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t run_decode_bs(const DecodeArgs& a, hipStream_t stream) {
  return a.block_size == 16 ? run_decode<T, D, 16>(a, stream) : run_decode<T, D, 32>(a, stream);
}

template <typename T>
hipError_t run_decode_d(const DecodeArgs& a, hipStream_t stream) {
  return a.head_dim == 64 ? run_decode_bs<T, 64>(a, stream) : run_decode_bs<T, 128>(a, stream);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  switch (a.dtype) {
    case PA_DTYPE_F32:
      return run_decode_d<F32>(a, stream);
    case PA_DTYPE_F16:
      return run_decode_d<F16>(a, stream);
    default:
      return run_decode_d<BF16>(a, stream);
  }
}

}  // namespace pa
