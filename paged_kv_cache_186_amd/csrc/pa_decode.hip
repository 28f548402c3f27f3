// Paged decode attention kernel for gfx950.
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
// (sequence, head), so it is HBM-bound and MFMA would idle; everything is built
// around streaming each (block, head) tile — BS*D contiguous elements, 4 KiB
// for fp16 D=128 BS=16 — with every lane moving 16 bytes per load, so one wave
// instruction covers 1 KiB of contiguous memory.
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
//
// Memory-level parallelism: each wave walks its tiles in groups of G and keeps
// the NEXT group's K/V loads in flight while it computes the current group
// (two register buffers), so up to 2*G tiles per wave are outstanding.
//
// Split-context merge without a second launch: a workgroup that covers one
// partition of a multi-partition context writes its partial (max, sum,
// unnormalised weighted V sum) to the workspace with L2-bypassing agent-scope
// stores and takes a ticket from the (sequence, head) counter; the workgroup
// that draws the last ticket merges all partials and resets the counter to
// zero for the next call.  (A device-scope fence would have to write back and
// invalidate the whole L2 of every XCD; the atomics avoid that.)

#include "pa_attend.h"
#include "pa_device.h"
#include "pa_internal.h"
#include "pagedattn.h"

namespace pa {
namespace {

// Launch shape; the defaults were chosen by measurement on MI355X and can be
// overridden at build time for tuning sweeps.
#ifndef PA_WAVES_PER_WG
#define PA_WAVES_PER_WG 4
#endif
#ifndef PA_TILES_PER_STAGE
#define PA_TILES_PER_STAGE 1
#endif
constexpr int kWavesPerGroup = PA_WAVES_PER_WG;  // waves per workgroup
constexpr int kTilesPerStage = PA_TILES_PER_STAGE;  // G: tiles per stage (2*G in flight per wave)

// G tiles' worth of K/V registers plus which logical block each one is (and,
// for an 8-bit cache, the tile's K and V scales).
template <typename T, int D, int BS, int G>
struct Stage {
  u32x4 k[G][Tile<T, D, BS>::kLoads];
  u32x4 v[G][Tile<T, D, BS>::kLoads];
  float sk[G], sv[G];
  int block[G];  // logical block index, or -1 when this slot holds no tile
};

// ---------------------------------------------------------------------------
// Log-sum-exp merge of one (sequence, head)'s partition partials, run by the
// workgroup that finished last.  With M = max_i m_i (base-2 units):
//   out = sum_i 2^(m_i - M) acc_i / sum_i 2^(m_i - M) l_i.
// All loads are agent-scope (coherent across XCDs) and independent, so they
// are issued in large batches: pass 1 streams (m_i, l_i) pairs and keeps an
// online (max, sum) per thread; pass 2 has every thread read a 16-byte slice
// of kMergeBatch partials before using any of them.
// ---------------------------------------------------------------------------
constexpr int kMergeCache = 1024;  // partitions whose weights are kept in LDS
constexpr int kMergeBatch = 16;    // partial slices in flight per thread

template <typename T, int D, int kThreads>
__device__ __forceinline__ void merge_partials(typename T::storage* __restrict__ out_row,
                               const float* __restrict__ ml,   // [nparts][2]
                               const float* __restrict__ acc,  // [nparts][D]
                               int nparts, float* s_w, float* s_red, float* s_pair) {
  const int t = threadIdx.x;
  // pass 1: global max and denominator; cache each partition's max
  float m = -INFINITY;
  float den = 0.f;
  for (int i = t; i < nparts; i += kThreads) {
    const uint64_t pr = load_coherent_u64(ml + 2 * i);
    const float mi = __builtin_bit_cast(float, static_cast<uint32_t>(pr));
    const float li = __builtin_bit_cast(float, static_cast<uint32_t>(pr >> 32));
    if (i < kMergeCache) s_w[i] = mi;
    lse_combine(m, den, mi, li);
  }
  // reduce (m, den) over the wave, then over the waves through LDS
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {
    const float m2 = __shfl_xor(m, off);
    const float d2 = __shfl_xor(den, off);
    lse_combine(m, den, m2, d2);
  }
  constexpr int kWaves = kThreads / kWave;
  if (t % kWave == 0) {
    s_pair[2 * (t / kWave)] = m;
    s_pair[2 * (t / kWave) + 1] = den;
  }
  __syncthreads();
  m = -INFINITY;
  den = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) lse_combine(m, den, s_pair[2 * w], s_pair[2 * w + 1]);
  const float M = m;
  for (int i = t; i < min(nparts, kMergeCache); i += kThreads) s_w[i] = fast_exp2(s_w[i] - M);
  __syncthreads();

  // pass 2: weighted sum of the partial vectors, 4 floats per thread per partial
  constexpr int kChunks = D / 4;             // 16-byte slices per partial row
  constexpr int kG = kThreads / kChunks;      // partials read side by side
  const int c = t % kChunks;
  const int g = t / kChunks;
  float num[4] = {0.f, 0.f, 0.f, 0.f};
  for (int i0 = g; i0 < nparts; i0 += kG * kMergeBatch) {
    uint64_t lo[kMergeBatch], hi[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const int i = min(i0 + u * kG, nparts - 1);  // clamped: always issue the load
      lo[u] = load_coherent_u64(acc + static_cast<size_t>(i) * D + 4 * c);
      hi[u] = load_coherent_u64(acc + static_cast<size_t>(i) * D + 4 * c + 2);
    }
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const int i = i0 + u * kG;
      float wi = 0.f;
      if (i < nparts) {
        wi = i < kMergeCache ? s_w[i]
                             : fast_exp2(__builtin_bit_cast(float, static_cast<uint32_t>(
                                             load_coherent_u64(ml + 2 * i))) - M);
      }
      num[0] = fmaf(wi, __builtin_bit_cast(float, static_cast<uint32_t>(lo[u])), num[0]);
      num[1] = fmaf(wi, __builtin_bit_cast(float, static_cast<uint32_t>(lo[u] >> 32)), num[1]);
      num[2] = fmaf(wi, __builtin_bit_cast(float, static_cast<uint32_t>(hi[u])), num[2]);
      num[3] = fmaf(wi, __builtin_bit_cast(float, static_cast<uint32_t>(hi[u] >> 32)), num[3]);
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) s_red[g * D + 4 * c + e] = num[e];
  __syncthreads();
  for (int d = t; d < D; d += kThreads) {
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < kG; ++k) sum += s_red[k * D + d];
    out_row[d] = T::pack(sum / den);
  }
}

// Grid: (head, partition, sequence); NW waves per workgroup.  Workgroup
// (h, p, s) covers blocks [p*PB, min((p+1)*PB, nblk)) of sequence s; wave w
// takes blocks w, w+NW, ... of that range.  QT: query / output storage; KT:
// K/V cache storage (QT itself, or an 8-bit type scaled per (block, head)).
// Query head h reads K/V head h / group (grouped-query attention; each query
// head reads its K/V head's tiles itself here — the balanced kernel is the
// one that shares a tile load between the heads of a group).
template <typename QT, typename KT, int D, int BS, int NW, int G>
__global__ __launch_bounds__(NW* kWave) void decode_kernel(
    typename QT::storage* __restrict__ out, uint32_t* __restrict__ counters,
    float* __restrict__ ws_ml, float* __restrict__ ws_acc, const typename QT::storage* __restrict__ q,
    const char* __restrict__ k_pool, const char* __restrict__ v_pool,
    const float* __restrict__ k_scales, const float* __restrict__ v_scales,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens,
    float q_scale, int num_heads, int num_kv_heads, int group, int num_blocks, int max_blocks,
    int part_blocks, int max_parts) {
  using C = Tile<KT, D, BS>;
  using St = Stage<KT, D, BS, G>;
  constexpr int E = KT::kElems;
  constexpr int kGroups = NW * C::kRowsPerLoad;
  __shared__ float s_m[kGroups];
  __shared__ float s_l[kGroups];
  __shared__ float s_acc[kGroups][D];
  __shared__ int s_bad[NW];
  __shared__ int s_last;
  __shared__ float s_w[kMergeCache];
  __shared__ float s_pair[2 * NW];
  static_assert(kGroups * D >= (NW * kWave / (D / 4)) * D, "merge reduction fits in s_acc");

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
      for (int d = threadIdx.x; d < D; d += blockDim.x) out[row * D + d] = QT::pack(0.f);
    return;
  }
  if (p >= nparts) return;

  const int kvh = h / group;  // K/V head read by query head h
  const int b_begin = p * part_blocks;
  const int b_end = min(nblk, b_begin + part_blocks);
  const int grp = lane / C::kLanesPerRow;
  const int col = lane % C::kLanesPerRow;

  float qf[E];
  QSlice<QT, KT>::load(q + row * D, col, qf);
#pragma unroll
  for (int e = 0; e < E; ++e) qf[e] *= q_scale;

  float m = -INFINITY;
  float l = 0.f;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  bool bad = false;

  const int32_t* tbl = block_tables + static_cast<size_t>(s) * max_blocks;
  const int first = b_begin + wave;
  const int nt = first < b_end ? (b_end - first + NW - 1) / NW : 0;  // tiles of this wave

  // Issue the K/V loads of tile k of this wave (k < nt).
  auto load_tile = [&](St& st, int g, int k) __attribute__((always_inline)) {
    const int j = first + k * NW;
    int phys = tbl[j];
    if (static_cast<unsigned>(phys) >= static_cast<unsigned>(num_blocks)) {
      bad = true;  // never dereference an id outside the pool
      phys = 0;
    }
    const size_t tile = (static_cast<size_t>(phys) * num_kv_heads + kvh) * C::kTileBytes;
    const char* kb = k_pool + tile + lane * kVecBytes;
    const char* vb = v_pool + tile + lane * kVecBytes;
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) st.k[g][i] = load16_stream(kb + i * C::kLoadBytes);
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) st.v[g][i] = load16_stream(vb + i * C::kLoadBytes);
    if constexpr (KT::kScaled) {
      st.sk[g] = load_uniform_f32(k_scales + static_cast<size_t>(phys) * num_kv_heads + kvh);
      st.sv[g] = load_uniform_f32(v_scales + static_cast<size_t>(phys) * num_kv_heads + kvh);
    } else {
      st.sk[g] = st.sv[g] = 1.f;
    }
    st.block[g] = j;
  };
  auto attend_slot = [&](const St& st, int g) __attribute__((always_inline)) {
    const int j = st.block[g];
    const int tok0 = j * BS + grp;
    if ((j + 1) * BS <= L)
      attend_tile<KT, D, BS, false>(st.k[g], st.v[g], qf, m, l, acc, tok0, L, st.sk[g], st.sv[g]);
    else
      attend_tile<KT, D, BS, true>(st.k[g], st.v[g], qf, m, l, acc, tok0, L, st.sk[g], st.sv[g]);
  };
  // A full stage holds G existing tiles: no per-slot guards, so every load it
  // issues is consumed on every path (the compiler then knows which loads are
  // outstanding and never waits on the prefetched stage early).
  auto load_full = [&](St& st, int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int g = 0; g < G; ++g) load_tile(st, g, k0 + g);
    // keep the scheduler from sinking these loads below the compute that
    // follows: they must be in flight while the previous stage is consumed
    __builtin_amdgcn_sched_barrier(0);
  };
  auto attend_full = [&](const St& st) __attribute__((always_inline)) {
#pragma unroll
    for (int g = 0; g < G; ++g) attend_slot(st, g);
  };

  // Steady state over the full stages: load b, compute a, load the next a,
  // compute b — no conditional load inside the loop, so at every point the
  // compiler knows exactly one prefetched stage is outstanding.  The epilogue
  // finishes the last one or two full stages, then the partial stage (fewer
  // than G tiles), if any.
  const int nfs = nt / G;
  St a, b;
  if (nfs > 0) load_full(a, 0);
  int st = 0;
  for (; st + 2 < nfs; st += 2) {
    load_full(b, (st + 1) * G);
    attend_full(a);
    load_full(a, (st + 2) * G);
    attend_full(b);
  }
  if (st + 1 < nfs) {
    load_full(b, (st + 1) * G);
    attend_full(a);
    attend_full(b);
  } else if (st < nfs) {
    attend_full(a);
  }
  if constexpr (G > 1) {
    const int rem = nt - nfs * G;
#pragma unroll
    for (int g = 0; g < G - 1; ++g)
      if (g < rem) load_tile(b, g, nfs * G + g);
#pragma unroll
    for (int g = 0; g < G - 1; ++g)
      if (g < rem) attend_slot(b, g);
  }

  // Merge the kGroups lane-group states of this workgroup through LDS.
  const int gidx = wave * C::kRowsPerLoad + grp;
  if (col == 0) {
    s_m[gidx] = m;
    s_l[gidx] = l;
  }
#pragma unroll
  for (int e = 0; e < E; ++e) s_acc[gidx][col * E + e] = acc[e];
  if (lane == 0) s_bad[wave] = bad ? 1 : 0;
  __syncthreads();

  const int d = threadIdx.x;  // blockDim.x >= D
  float M = -INFINITY;
  float lsum = 0.f;
  float o = 0.f;
  if (d < D) {
    int any_bad = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) any_bad |= s_bad[w];
#pragma unroll
    for (int k = 0; k < kGroups; ++k) M = fmaxf(M, s_m[k]);
#pragma unroll
    for (int k = 0; k < kGroups; ++k) {
      const float a_k = fast_exp2(s_m[k] - M);  // groups that met no token: exp2(-inf) = 0
      lsum = fmaf(a_k, s_l[k], lsum);
      o = fmaf(a_k, s_acc[k][d], o);
    }
    if (any_bad) {
      o = __builtin_nanf("");
      lsum = __builtin_nanf("");
    }
  }
  if (nparts == 1) {
    if (d < D) out[row * D + d] = QT::pack(o / lsum);
    return;
  }

  // Publish this partition's partial, then take a ticket.  Partials are
  // written and read with agent-scope atomic accesses: on gfx950 these bypass
  // the per-XCD L2 (which is not coherent across XCDs), so no L2 write-back or
  // invalidate is needed — a device-scope fence would flush the whole L2 of
  // every XCD once per workgroup.  Ordering comes from completion: the barrier
  // waits until this workgroup's partial stores are performed (s_waitcnt)
  // before thread 0 takes the ticket, and the last workgroup issues its partial
  // loads only after its ticket has returned.
  const size_t base = row * max_parts;
  if (d < D) {
    __hip_atomic_store(&ws_acc[(base + p) * D + d], o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (d == 0) {
      __hip_atomic_store(&ws_ml[(base + p) * 2 + 0], M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&ws_ml[(base + p) * 2 + 1], lsum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // Wait until this wave's partial stores are performed (a workgroup barrier
  // alone does not wait for global stores); the clobber keeps the compiler
  // from moving memory accesses across the wait.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t ticket =
        __hip_atomic_fetch_add(&counters[row], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (ticket == static_cast<uint32_t>(nparts - 1));
  }
  __syncthreads();
  if (!s_last) return;

  // Last arrival: merge every partition of this (s, h).  s_acc is free again
  // and serves as the reduction buffer.
  merge_partials<QT, D, NW * kWave>(out + row * D, ws_ml + base * 2, ws_acc + base * D, nparts,
                                   s_w, &s_acc[0][0], s_pair);
  if (threadIdx.x == 0)  // ready for the next call
    __hip_atomic_store(&counters[row], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One workgroup per CU when each streams much and there are many: with up
// to four resident per CU the older one is served first and the rest trail;
// reserving more than half the CU's LDS (dynamic LDS, unused) leaves room for
// one.  Measured, one per CU against four: 512-token partitions of a 16-bit
// D = 128 cache (256 KiB of K and V per workgroup) over 4 x 131072 tokens
// 1507 -> 1317 us (1436 -> 1322 on another box), over 1 x 131072 367 -> 350
// us; but with less per workgroup it loses — the same over an 8-bit cache 188
// -> 247 us, 256-token partitions 370 -> 397 us, the layer shape with
// 64-token partitions 27.8 -> 46.5 us — and so it does where most partitions
// are empty (continuous batching, 512-token partitions of a 129-block table:
// 142 -> 155 us).  Hence: at least kPartOneWgBytes of K and V per partition
// and at least kPartOneWgMinParts partitions per row.
constexpr size_t kPartOneWgBytes = 256 * 1024;
constexpr int kPartOneWgMinParts = 32;
constexpr size_t kPartOneWgLds = 96 * 1024;

template <typename QT, typename KT, int D, int BS>
hipError_t run_decode(const DecodeArgs& a, hipStream_t stream) {
  using S = typename QT::storage;
  const dim3 grid(a.num_heads, a.max_partitions, a.num_seqs);
  // K and V bytes of one (head, partition)
  const size_t part_bytes = static_cast<size_t>(a.partition_blocks) * BS * D * sizeof(typename KT::storage) * 2;
  const size_t dyn_lds =
      (a.max_partitions >= kPartOneWgMinParts && part_bytes >= kPartOneWgBytes) ? kPartOneWgLds : 0;
  hipLaunchKernelGGL((decode_kernel<QT, KT, D, BS, kWavesPerGroup, kTilesPerStage>), grid,
                     dim3(kWavesPerGroup * kWave), dyn_lds, stream, static_cast<S*>(a.out), a.counters,
                     a.ws_ml, a.ws_acc, static_cast<const S*>(a.q),
                     static_cast<const char*>(a.k_pool), static_cast<const char*>(a.v_pool),
                     a.k_scales, a.v_scales, a.block_tables, a.context_lens, a.scale * kLog2e,
                     a.num_heads, a.num_kv_heads, a.num_heads / a.num_kv_heads, a.num_blocks,
                     a.max_blocks_per_seq, a.partition_blocks, a.max_partitions);
  return hipGetLastError();
}

template <typename QT, typename KT, int D>
hipError_t run_decode_bs(const DecodeArgs& a, hipStream_t stream) {
  return a.block_size == 16 ? run_decode<QT, KT, D, 16>(a, stream) : run_decode<QT, KT, D, 32>(a, stream);
}

template <typename QT, typename KT>
hipError_t run_decode_d(const DecodeArgs& a, hipStream_t stream) {
  return a.head_dim == 64 ? run_decode_bs<QT, KT, 64>(a, stream) : run_decode_bs<QT, KT, 128>(a, stream);
}

template <typename QT>
hipError_t run_decode_kv(const DecodeArgs& a, hipStream_t stream) {
  switch (a.kv_dtype) {
    case PA_DTYPE_FP8_E4M3:
      return run_decode_d<QT, FP8E4M3>(a, stream);
    case PA_DTYPE_FP8_E5M2:
      return run_decode_d<QT, FP8E5M2>(a, stream);
    default:
      return run_decode_d<QT, QT>(a, stream);
  }
}

}  // namespace

hipError_t launch_decode_partitioned(const DecodeArgs& a, hipStream_t stream) {
  switch (a.dtype) {
    case PA_DTYPE_F32:
      return run_decode_d<F32, F32>(a, stream);
    case PA_DTYPE_F16:
      return run_decode_kv<F16>(a, stream);
    default:
      return run_decode_kv<BF16>(a, stream);
  }
}

}  // namespace pa
