// Attention of many query rows per sequence (chunked prefill) over the paged
// KV cache on the matrix cores (gfx950 MFMA), with the keys and values of
// each step staged in LDS once per workgroup.
//
// What is computed is what prefill_kernel computes: for every sequence s, its
// last Tq_s tokens attend causally over its cache — query token i at position
// p = L_s - Tq_s + i sees the keys at positions 0..p — and query head h reads
// K/V head h / G (page "mlx-paged-attention: Bringing vLLM-level High
// Throughput Inference to Apple Silicon", comparison with vLLM and future
// plans; the attention itself is the ordinary softmax attention read through
// the block table, vLLM tutorial page "3. PagedAttention原理", §3.2 and the
// closing remarks of §3.4).
//
// This kernel serves the shapes where the query rows alone fill the GPU (the
// library's default split keeps every row in one partition): the rows of one
// (sequence, K/V head) — (query token, head of the group) pairs, token-major
// — are cut into blocks of 128, and a workgroup of four waves takes one block
// (32 rows per wave, two 16-row MFMA tiles).  The keys are walked in steps of
// 64: each step's K and V rows (2 x 16 KiB at D = 128) are copied from HBM
// straight into LDS by the direct global-to-LDS loads of gfx950 (no
// registers: global_load_lds_dwordx4, 1 KiB per wave instruction, 16 bytes
// per lane) into one of two stages while the other step is computed; all
// four waves read their MFMA operands from there, so every K/V byte reaches
// the CU once per 128 query rows instead of once per 16 or 32.  In LDS, the
// 16-byte chunk c of key k sits at position c ^ swz(k) of its row, so that
// the keys an operand read touches fall on different banks.
//
// Per step and wave (32 rows, 64 keys):
//   S^T = K Q^T     per 16-key block and 32-element slice one
//                   v_mfma_f32_16x16x32 per tile (A = 16 keys x 32 elements
//                   from LDS, shared by the two tiles; B = the tile's queries,
//                   in registers for the whole block);
//   softmax         the lane's 16 scores per tile, the row's maximum over its
//                   four lanes, rescaling deferred until it grows by 2^8;
//                   causal and context masks only on the steps that cross a
//                   row's position;
//   O^T += V^T P^T  per 32 keys and 16-value tile one product per tile (A =
//                   V transposed, from LDS by two transposing reads, shared
//                   by the tiles), plus one with every value 1 for the row
//                   sums.
// Items (sequence, K/V head, row block) run in that order, the blocks of one
// (sequence, K/V head) latest rows first, and consecutive items on one XCD,
// so that the blocks reading the same keys share that XCD's L2.

#include "pa_attend.h"
#include "pa_device.h"
#include "pa_internal.h"
#include "pa_mfma.h"
#include "pagedattn.h"

namespace pa {
namespace {

typedef __attribute__((address_space(1))) void global_void_t;
typedef __attribute__((address_space(3))) void lds_void_t;

#ifndef PA_PREFILL_TILE_KEYS
#define PA_PREFILL_TILE_KEYS 64
#endif
constexpr int kTlWaves = 4;
constexpr int kTlTiles = 2;                      // 16-row tiles per wave
constexpr int kTlRows = kTlWaves * kTlTiles * 16;  // rows per workgroup (128)
constexpr int kTlKeys = PA_PREFILL_TILE_KEYS;    // keys per step (32 or 64)
constexpr int kTlKB = kTlKeys / 16;              // 16-key blocks per step
constexpr int kTlWaveKeys = kTlKeys / 4;         // keys of a step one wave loads

typedef __attribute__((address_space(3))) s4_t lds_s4_t;

// one 16-byte direct global-to-LDS load per lane: the wave's 64 lanes fill
// the 1 KiB at lds (a wave-uniform address) in lane order
__device__ __forceinline__ void load_lds16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((global_void_t*)(g), (lds_void_t*)(lds), 16, 0, 0);
}
// the same with 4 bytes per lane (256 bytes per wave instruction)
__device__ __forceinline__ void load_lds4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((global_void_t*)(g), (lds_void_t*)(lds), 4, 0, 0);
}

// Workgroup barrier for the steps.  A memory fence (as in __syncthreads())
// would make every wave wait for all of its loads in flight, the next step's
// direct loads among them (they write LDS); instead each wave completes its
// own LDS accesses (lgkmcnt) and its direct loads of the step being entered
// (an explicit vmcnt before the barrier), and the empty asm statements keep
// the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <typename T, int D, int BS>
__global__ __launch_bounds__(kTlWaves* kWave, 2) void prefill_tile_kernel(
    typename T::storage* __restrict__ out, const typename T::storage* __restrict__ q,
    const char* __restrict__ k_pool, const char* __restrict__ v_pool, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ query_start, float qk_scale,
    uint32_t q_sign_bits, int num_seqs, int num_rows, int num_heads, int num_kv_heads, int num_blocks,
    int max_blocks, int max_items) {
  using S16 = typename T::storage;
  using M = Mfma<T>;
  using PV = PvOps<T, 2>;
  using pw_t = typename PV::word_t;
  constexpr int kThreads = kTlWaves * kWave;
  constexpr int kRowB = D * 2;                       // bytes of one K or V row
  constexpr int kCpr = kRowB / 16;                   // 16-byte chunks per row (16 or 8)
  constexpr int kRowsPer256 = 256 / kRowB;           // rows per 256 bytes of LDS banks (1 or 2)
  constexpr int kStepB = kTlKeys * kRowB;            // bytes of one step's K (or V) rows
  constexpr int kUnits = kStepB / 1024 / kTlWaves;   // 1 KiB loads per wave and matrix per step
  static_assert(kUnits * 1024 * kTlWaves == kStepB, "whole 1 KiB loads");
  static_assert(kUnits * 1024 / kRowB == kTlWaveKeys, "each wave loads a quarter of a step");
  constexpr int kSl = D / 32;                        // 32-element slices of the S^T contraction
  // chunk swizzles (16-byte chunk c of key k sits at position c ^ swz(k)):
  // K operands read the same chunk of 16 keys, which must fall on distinct
  // banks; V reads read 2 chunks of 4 consecutive keys, 8 distinct chunks
  auto swz_k = [](int k) { return (k / kRowsPer256) % kCpr; };
  auto swz_v = [](int k) { return 2 * (k & 3); };
  constexpr int kDt = D / 16;                        // 16-element value tiles (rows of the P.V A operand)
  constexpr int kPer = (kPfMaxSeqs + kThreads - 1) / kThreads;
  // two steps in flight, each stage a separate array (K and V)
  __shared__ __attribute__((aligned(1024))) char s_k0[kStepB];
  __shared__ __attribute__((aligned(1024))) char s_v0[kStepB];
  __shared__ __attribute__((aligned(1024))) char s_k1[kStepB];
  __shared__ __attribute__((aligned(1024))) char s_v1[kStepB];
  __shared__ int s_off[kPfMaxSeqs + 1];  // items of the sequences before s
  __shared__ int s_wsum[kTlWaves];
  // per stage and wave: the wave's block id of the step was outside the pool
  __shared__ __attribute__((aligned(16))) int s_bad[2][kTlWaves];
  // per wave two windows of 64 block-table entries (see issue_step)
  __shared__ __attribute__((aligned(256))) int s_tbl[kTlWaves][2][kWave];
  static_assert(kTlWaves == 4, "s_bad read as one 16-byte vector");

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int S = num_seqs;
  const int HKV = num_kv_heads;
  const int G = num_heads / num_kv_heads;
  const int cap = max_blocks * BS;

  // 1. items per sequence (K/V heads x 128-row blocks) and their prefix sum;
  //    query bounds clamped to the q / out rows
  int cnt[kPer];
  int mine = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int s = tid * kPer + i;
    int c = 0;
    if (s < S) {
      const int q0 = min(max(query_start[s], 0), num_rows);
      const int q1 = min(max(query_start[s + 1], 0), num_rows);
      const int rows = max(q1 - q0, 0) * G;
      c = HKV * ((rows + kTlRows - 1) / kTlRows);
    }
    cnt[i] = c;
    mine += c;
  }
  const int incl = wave_prefix_sum(mine);
  if (lane == kWave - 1) s_wsum[wave] = incl;
  __syncthreads();
  int run = incl - mine;
  int total = 0;
#pragma unroll
  for (int w = 0; w < kTlWaves; ++w) {
    run += (w < wave) ? s_wsum[w] : 0;
    total += s_wsum[w];
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int s = tid * kPer + i;
    if (s < S) s_off[s] = run;
    run += cnt[i];
  }
  __syncthreads();
  total = min(__builtin_amdgcn_readfirstlane(total), max_items);

  const u32x4 q_sign = {q_sign_bits, q_sign_bits, q_sign_bits, q_sign_bits};
  const int col = lane % 16;
  const int g4 = lane / 16;

  for (int item = xcd_local_index(blockIdx.x, gridDim.x); item < total; item += gridDim.x) {
    // 2. (sequence, K/V head, row block)
    int lo = 0;
    int hi = S - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_off[mid] <= item)
        lo = mid;
      else
        hi = mid - 1;
    }
    const int s = __builtin_amdgcn_readfirstlane(lo);
    const int L = min(max(context_lens[s], 0), cap);
    const int q0 = min(max(query_start[s], 0), num_rows);
    const int Tq = max(min(max(query_start[s + 1], 0), num_rows) - q0, 0);
    const int Mrows = Tq * G;
    const int nb = (Mrows + kTlRows - 1) / kTlRows;
    const int local = item - __builtin_amdgcn_readfirstlane(s_off[s]);
    const int kvh = local / nb;
    const int rb = nb - 1 - (local - kvh * nb);  // latest rows (most keys) first
    const int first = L - Tq;                      // position of query token 0

    // this lane's rows (one per tile) and the positions they see up to
    int tok[kTlTiles], head[kTlTiles], pos[kTlTiles], tile_max[kTlTiles];
    bool ok[kTlTiles];
#pragma unroll
    for (int t = 0; t < kTlTiles; ++t) {
      const int r0 = rb * kTlRows + wave * 32 + 16 * t;  // the tile's first row
      const int r = r0 + col;
      ok[t] = r < Mrows;
      tok[t] = r / G;
      head[t] = kvh * G + (r - tok[t] * G);
      pos[t] = ok[t] ? first + tok[t] : -1;
      tile_max[t] = (r0 < Mrows) ? first + (min(Mrows, r0 + 16) - 1) / G : -1;
    }
    const int wave_max = max(tile_max[0], tile_max[1]);
    const int wave_min = (rb * kTlRows + wave * 32 < Mrows) ? first + (rb * kTlRows + wave * 32) / G : INT_MAX;
    // keys the block needs: through the position of its last row
    const int n_keys = min(L, first + (min(Mrows, (rb + 1) * kTlRows) - 1) / G + 1);
    const int n_steps = n_keys > 0 ? (n_keys + kTlKeys - 1) / kTlKeys : 0;

    f4_t acc[kTlTiles][kDt];
    f4_t lacc[kTlTiles];
    float m[kTlTiles];
#pragma unroll
    for (int t = 0; t < kTlTiles; ++t) {
      m[t] = -INFINITY;
      lacc[t] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt) acc[t][dt] = f4_t{0.f, 0.f, 0.f, 0.f};
    }
    bool bad[kTlTiles] = {false, false};

    if (n_steps > 0) {
      // the queries (B operands of S^T), a negative scale flipping their signs
      u32x4 qv[kTlTiles][kSl];
#pragma unroll
      for (int t = 0; t < kTlTiles; ++t) {
        const S16* qr = q + (static_cast<size_t>(q0 + tok[t]) * num_heads + head[t]) * D + 8 * g4;
#pragma unroll
        for (int sl = 0; sl < kSl; ++sl)
          qv[t][sl] = ok[t] ? (load16(qr + 32 * sl) ^ q_sign) : u32x4{0u, 0u, 0u, 0u};
      }

      // block-table entries in windows of 64, copied by direct loads into
      // the wave's two LDS slots: window w (entries 64 w .. 64 w + 63) in slot
      // w % 2.  A wave asks for non-decreasing blocks, so when it enters
      // window w the slot of window w - 1 takes window w + 1, which is needed
      // at least 16 steps later: by then the step waits have completed it.
      const int32_t* tbl = block_tables + static_cast<size_t>(s) * max_blocks;
      auto load_window = [&](int w) __attribute__((always_inline)) {
        load_lds4(tbl + min(w * kWave + lane, max_blocks - 1), s_tbl[wave][w & 1]);
      };
      int win = 0;
      load_window(0);
      load_window(1);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

      // Step c's K (or V) rows, loaded directly into its stage: wave w loads
      // keys 16 w .. 16 w + 15 of the step (one block: BS >= 16 and the keys
      // 16-aligned); keys past n_keys load key n_keys - 1 instead (finite;
      // masked).  The K loads also look up the wave's block and record
      // whether its id was outside the pool; the V loads of the step reuse
      // the block.
      size_t row0 = 0;  // first pool row of the wave's block for the step being loaded
      auto issue_rows = [&](int c, const char* pool, char* stage_base, bool is_v, int stage)
          __attribute__((always_inline)) {
        const bool lookup = !is_v;
        const int c0 = c * kTlKeys;
        if (lookup) {
          const int kw = min(c0 + kTlWaveKeys * wave, n_keys - 1);
          const int b = kw / BS;
          if ((b >> 6) != win) {
            win = b >> 6;
            load_window(win + 1);
          }
          int phys = __builtin_amdgcn_readfirstlane(s_tbl[wave][win & 1][b & (kWave - 1)]);
          const bool out_of_pool = static_cast<unsigned>(phys) >= static_cast<unsigned>(num_blocks);
          if (out_of_pool) phys = 0;  // never dereference an id outside the pool
          if (lane == 0) s_bad[stage][wave] = out_of_pool ? 1 : 0;
          row0 = (static_cast<size_t>(phys) * HKV + kvh) * BS;
        }
#pragma unroll
        for (int u = 0; u < kUnits; ++u) {
          const int slot = (wave * kUnits + u) * kWave + lane;  // 16-byte slot of the step's rows
          const int kk = slot / kCpr;
          const int cg = (slot % kCpr) ^ (is_v ? swz_v(kk) : swz_k(kk));  // the chunk stored in that slot
          const int key = min(c0 + kk, n_keys - 1);
          load_lds16(pool + (row0 + key % BS) * kRowB + cg * 16, stage_base + (wave * kUnits + u) * 1024);
        }
      };

      // LDS byte offsets of the lane's operands within a stage.  K (read
      // by ds_read_b128): key 16 kb + col, elements 32 sl + 8 g4 ..; its
      // swizzle does not depend on kb (16 keys span whole 256-byte bank
      // rows), so one offset per slice serves every block.  V (read by
      // ds_read_b64_tr_b16, see below): key 4 g4 + (col / 4) of each 16-key
      // block, values 16 dt + 4 (col % 4) ..; one offset per value tile.
      int koff[kSl];
      int voff[kDt];
#pragma unroll
      for (int sl = 0; sl < kSl; ++sl) koff[sl] = col * kRowB + (((4 * sl + g4) ^ swz_k(col)) * 16);
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt) {
        const int kk = 4 * g4 + col / 4;
        voff[dt] = kk * kRowB + (((2 * dt + (col % 4) / 2) ^ swz_v(kk)) * 16) + 8 * (col % 2);
      }

      // 3. the steps.  A read of LDS after a direct load was issued waits
      //    for every direct load in flight (the compiler cannot tell the
      //    stages apart), so a step reads its K operands in one batch,
      //    issues the next step's loads (into the other stage) and runs S^T
      //    and the softmax on registers while they land; its V reads, slice
      //    by slice between the P.V products, come after.  The barrier at the
      //    top of a step follows every wave's wait for its own loads of that
      //    step.
      issue_rows(0, k_pool, s_k0, false, 0);
      issue_rows(0, v_pool, s_v0, true, 0);
      for (int c = 0; c < n_steps; ++c) {
        const int stage = c & 1;
        const char* sk = stage ? s_k1 : s_k0;
        const char* sv = stage ? s_v1 : s_v0;
        char* nk = stage ? s_k0 : s_k1;
        char* nv = stage ? s_v0 : s_v1;
        const bool next = c + 1 < n_steps;
        const int c0 = c * kTlKeys;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_barrier();
        // a block id outside the pool poisons the tiles that see its keys
        const u32x4 sb = *reinterpret_cast<const u32x4*>(s_bad[stage]);
#pragma unroll
        for (int w = 0; w < kTlWaves; ++w)
#pragma unroll
          for (int t = 0; t < kTlTiles; ++t) bad[t] = bad[t] || (sb[w] != 0u && c0 + kTlWaveKeys * w <= tile_max[t]);
        // (a wave whose rows all end before c0 still runs the step: its
        // scores are all masked, so nothing changes, and one path through the
        // loop keeps the accumulators in place)
        // the K operands of the step (16 keys x 32 elements per block and
        // slice), then the next step's loads, then S^T
        u32x4 ka[kSl][kTlKB];
#pragma unroll
        for (int sl = 0; sl < kSl; ++sl)
#pragma unroll
          for (int kb = 0; kb < kTlKB; ++kb)
            ka[sl][kb] = *reinterpret_cast<const u32x4*>(sk + koff[sl] + kb * 16 * kRowB);
        if (next) {
          issue_rows(c + 1, k_pool, nk, false, stage ^ 1);
          issue_rows(c + 1, v_pool, nv, true, stage ^ 1);
        }
        f4_t sc[kTlTiles][kTlKB];
#pragma unroll
        for (int t = 0; t < kTlTiles; ++t)
#pragma unroll
          for (int kb = 0; kb < kTlKB; ++kb) sc[t][kb] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sl = 0; sl < kSl; ++sl)
#pragma unroll
          for (int kb = 0; kb < kTlKB; ++kb)
#pragma unroll
            for (int t = 0; t < kTlTiles; ++t) sc[t][kb] = M::qk(ka[sl][kb], qv[t][sl], sc[t][kb]);
        // softmax; lane l holds keys c0 + 16 kb + 4 g4 + i of row col.  Only
        // the steps that reach past a row's position (the last one or two of
        // a block) mask: the others take a path without selects.
        const bool masked = c0 + kTlKeys - 1 > wave_min;
        if (masked) {
#pragma unroll
          for (int t = 0; t < kTlTiles; ++t)
#pragma unroll
            for (int kb = 0; kb < kTlKB; ++kb)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (c0 + 16 * kb + 4 * g4 + i > pos[t]) sc[t][kb][i] = -INFINITY;
        }
        pw_t pw[kTlTiles][kTlKB / 2];
        bool grow = false;
        float cms[kTlTiles];
#pragma unroll
        for (int t = 0; t < kTlTiles; ++t) {
          float cm = -INFINITY;
#pragma unroll
          for (int kb = 0; kb < kTlKB; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) cm = fmaxf(cm, sc[t][kb][i]);
          cm = fold_max<16>(cm);  // the row's four lanes
          cms[t] = (cm == -INFINITY) ? -INFINITY : cm * qk_scale;
          grow = grow || (cms[t] > m[t] + kRescaleLog2);
        }
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
          for (int t = 0; t < kTlTiles; ++t) {
            const float mn = fmaxf(m[t], cms[t]);
            const float alpha = (m[t] == -INFINITY) ? 0.f : fast_exp2(m[t] - mn);
            lacc[t] *= alpha;
#pragma unroll
            for (int dt = 0; dt < kDt; ++dt) acc[t][dt] *= alpha;
            m[t] = mn;
          }
        }
#pragma unroll
        for (int t = 0; t < kTlTiles; ++t) {
          const float nm = -m[t];
          float p[kTlKB][4];
          if (masked) {  // masked keys, and rows that have seen no key yet (m = -inf), give 0
#pragma unroll
            for (int kb = 0; kb < kTlKB; ++kb)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                p[kb][i] = (sc[t][kb][i] == -INFINITY) ? 0.f : fast_exp2(fmaf(sc[t][kb][i], qk_scale, nm));
          } else {
#pragma unroll
            for (int kb = 0; kb < kTlKB; ++kb)
#pragma unroll
              for (int i = 0; i < 4; ++i) p[kb][i] = fast_exp2(fmaf(sc[t][kb][i], qk_scale, nm));
          }
#pragma unroll
          for (int h = 0; h < kTlKB / 2; ++h)
            pw[t][h] = pw_t{M::pack2(p[2 * h][0], p[2 * h][1]), M::pack2(p[2 * h][2], p[2 * h][3]),
                            M::pack2(p[2 * h + 1][0], p[2 * h + 1][1]), M::pack2(p[2 * h + 1][2], p[2 * h + 1][3])};
        }
        // O^T += V^T P^T per 32 keys (blocks 2 h, 2 h + 1) and 16-value tile
        // dt.  The A operand (V transposed: 16 values x 32 keys) comes from two
        // transposing reads: in each group of 16 lanes, lane 4 j + a reads 4
        // values (16 dt + 4 a ..) of key j of the group's four, and the read
        // hands lane 4 a + b value 16 dt + 4 a + b of all four keys — lane l
        // gets value 16 dt + l % 16 of keys 4 (l / 16) + j of the block, the
        // keys its P operand holds.  Reads run one tile ahead.
        auto load_v = [&](int j, u32x4& dst) __attribute__((always_inline)) {
          const int h = j / kDt;
          const int dt = j % kDt;
          const s4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s4_t*)(sv + voff[dt] + 32 * h * kRowB));
          const s4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s4_t*)(sv + voff[dt] + (32 * h + 16) * kRowB));
          const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
          const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
          dst = u32x4{l2.x, l2.y, h2.x, h2.y};
        };
        u32x4 va[2];
        load_v(0, va[0]);
#pragma unroll
        for (int j = 0; j < kTlKB / 2 * kDt; ++j) {
          const int h = j / kDt;
          const int dt = j % kDt;
          if (j + 1 < kTlKB / 2 * kDt) load_v(j + 1, va[(j + 1) & 1]);
#pragma unroll
          for (int t = 0; t < kTlTiles; ++t) acc[t][dt] = PV::mma(va[j & 1], pw[t][h], acc[t][dt]);
          if (dt == kDt - 1) {
            const pw_t ones = {M::kOnes, M::kOnes, M::kOnes, M::kOnes};
#pragma unroll
            for (int t = 0; t < kTlTiles; ++t) lacc[t] = PV::mma(ones, pw[t][h], lacc[t]);
          }
        }
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }

    // 4. the rows: lane l holds row col's values 16 dt + 4 g4 + i in
    //    acc[t][dt][i]; a row that sees no key is zero
#pragma unroll
    for (int t = 0; t < kTlTiles; ++t) {
      if (!ok[t]) continue;
      float lrow = lacc[t][0];
      if (bad[t]) lrow = __builtin_nanf("");
      const float inv = (lrow == 0.f) ? 0.f : 1.f / lrow;
      S16* orow = out + (static_cast<size_t>(q0 + tok[t]) * num_heads + head[t]) * D + 4 * g4;
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt)
        *reinterpret_cast<u32x2*>(orow + 16 * dt) =
            u32x2{M::pack2(acc[t][dt][0] * inv, acc[t][dt][1] * inv), M::pack2(acc[t][dt][2] * inv, acc[t][dt][3] * inv)};
    }
    __syncthreads();  // the stages and s_bad are free for the next item
  }
}
template <typename T, int D, int BS>
hipError_t run_tiles(const PrefillArgs& a, hipStream_t stream) {
  using S16 = typename T::storage;
  hipLaunchKernelGGL((prefill_tile_kernel<T, D, BS>), dim3(a.workgroups), dim3(kTlWaves * kWave), 0, stream,
                     static_cast<S16*>(a.out), static_cast<const S16*>(a.q), static_cast<const char*>(a.k_pool),
                     static_cast<const char*>(a.v_pool), a.block_tables, a.context_lens, a.query_start,
                     fabsf(a.scale) * kLog2e, a.scale < 0.f ? 0x80008000u : 0u, a.num_seqs, a.num_query_rows,
                     a.num_heads, a.num_kv_heads, a.num_blocks, a.max_blocks_per_seq, a.max_items);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t run_tiles_bs(const PrefillArgs& a, hipStream_t stream) {
  return a.block_size == 16 ? run_tiles<T, D, 16>(a, stream) : run_tiles<T, D, 32>(a, stream);
}

template <typename T>
hipError_t run_tiles_d(const PrefillArgs& a, hipStream_t stream) {
  return a.head_dim == 64 ? run_tiles_bs<T, 64>(a, stream) : run_tiles_bs<T, 128>(a, stream);
}

}  // namespace

hipError_t launch_prefill_tiles(const PrefillArgs& a, hipStream_t stream) {
  return a.dtype == PA_DTYPE_BF16 ? run_tiles_d<BF16>(a, stream) : run_tiles_d<F16>(a, stream);
}

}  // namespace pa
